"""The differentiable entry points (flash_attention, scaled_dot_product_attention)
on the GPU: outputs and gradients through torch.autograd equal the direct
attn_fwd / attn_bwd calls bit for bit, and agree with the fp64 oracles."""

import numpy as np
import pytest

import exact_attention_121_amd as ea
from exact_attention_121_amd.inputs import make_qkv
from oracle.attention import attention_ref
from oracle.backward import attention_bwd_ref
from parity_util import assert_parity, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(1, 4, 2, 300, 128, True), (2, 2, 2, 129, 64, False), (1, 8, 1, 257, 256, True), (1, 2, 2, 100, 96, False)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("entry", ["flash_attention", "sdpa"])
def test_autograd_matches_direct_calls_and_oracle(shape, entry):
    import torch

    from test_gpu_backward import assert_grad_parity, make_dout

    B, Hq, Hkv, N, d, causal = shape
    print(f"[autograd] {entry} {shape}", flush=True)
    qn, kn, vn = make_qkv(B, Hq, Hkv, N, d, seed=31 + N + d)
    don = make_dout(qn.shape, seed=37 + N)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v, do = to_dev(qn, kn, vn, don)
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    if entry == "flash_attention":
        o = ea.flash_attention(q, k, v, attn_scale=scale, causal=causal)
    else:
        o = ea.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    o.backward(do)
    torch.cuda.synchronize()

    with torch.no_grad():
        o_ref, lse = ea.attn_fwd(q.detach(), k.detach(), v.detach(), scale=scale, causal=causal)
        grads = ea.attn_bwd(q.detach(), k.detach(), v.detach(), o_ref, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for name, a, b in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), grads):
        assert torch.equal(a, b), name

    O, L = attention_ref(qn, kn, vn, scale, causal=causal)
    assert_parity(o.detach().cpu().numpy(), None, O, L, what=f"{entry} {shape}")
    ref = attention_bwd_ref(qn, kn, vn, don, scale, causal=causal)
    assert_grad_parity([x.cpu().numpy() for x in (q.grad, k.grad, v.grad)], ref, f"{entry} {shape}")


def test_default_scale_and_bf16():
    import torch

    qn, kn, vn = make_qkv(1, 2, 1, 200, 128, seed=41)
    q, k, v = (t.to(torch.bfloat16).requires_grad_(True) for t in to_dev(qn, kn, vn))
    o = ea.flash_attention(q, k, v, causal=True)   # attn_scale defaults to 1/sqrt(d)
    o.float().sum().backward()
    torch.cuda.synchronize()
    with torch.no_grad():
        o_ref, _ = ea.attn_fwd(q.detach(), k.detach(), v.detach(), causal=True)
    assert o.dtype == torch.bfloat16 and torch.equal(o.detach(), o_ref)
    assert all(t.grad is not None and torch.isfinite(t.grad.float()).all() for t in (q, k, v))
