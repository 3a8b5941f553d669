"""Differentiable entry points over the fused kernels (argument marshalling only).

    o = flash_attention(q, k, v, attn_scale=None, causal=False)
    o = scaled_dot_product_attention(q, k, v, attn_mask=None, dropout_p=0.0,
                                     is_causal=False, scale=None)

The pages call the fused operator from PyTorch under these two names
([FA-Dict] section "calling": flash_attention with an attn_scale argument;
[CANN-FA] section "calling from PyTorch": scaled_dot_product_attention with
is_causal).  Both run attn_fwd in the forward and attn_bwd in the backward
(torch.autograd.Function), saving q, k, v, O and the LSE in between; every
product and reduction runs in the HIP kernels.  The tensors follow attn_fwd's
contract ([B, H, N, d], contiguous fp16 or bf16 on one AMD GPU, Hq a multiple
of Hkv); an upstream gradient that is not contiguous is copied to a contiguous
one.  What the kernels do not compute is refused, not emulated: an attention
mask other than None, dropout, or enable_gqa=False with Hq != Hkv.
"""

from __future__ import annotations

from .binding import attn_bwd, attn_fwd

_function = None


def _attention_function():
    """The torch.autograd.Function, built on first use (torch is imported
    lazily, like the rest of the binding)."""
    global _function
    if _function is None:
        import torch

        class FusedAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal):
                o, lse = attn_fwd(q, k, v, scale=scale, causal=causal)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.scale, ctx.causal = scale, causal
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), scale=ctx.scale, causal=ctx.causal)
                return dq, dk, dv, None, None

        _function = FusedAttention
    return _function


def flash_attention(q, k, v, attn_scale: float | None = None, causal: bool = False):
    """softmax(attn_scale * q k^T [+ causal mask]) v, differentiable in q, k
    and v.  attn_scale defaults to 1 / sqrt(d)."""
    return _attention_function().apply(q, k, v, attn_scale, bool(causal))


def scaled_dot_product_attention(q, k, v, attn_mask=None, dropout_p: float = 0.0, is_causal: bool = False,
                                 scale: float | None = None, enable_gqa: bool = True):
    """The fused kernels under torch's scaled_dot_product_attention signature
    (same meaning of scale and is_causal; [B, H, N, d] layout).  K/V heads
    fewer than the query heads are grouped (GQA/MQA) unless enable_gqa is
    False, which then requires equal head counts."""
    if attn_mask is not None:
        raise NotImplementedError("attn_mask is not supported: only the causal mask (is_causal=True) is fused")
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    if not enable_gqa and q.shape[1] != k.shape[1]:
        raise ValueError("q and k have different head counts and enable_gqa is False")
    return _attention_function().apply(q, k, v, scale, bool(is_causal))
