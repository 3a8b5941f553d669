"""Fused exact attention for AMD Instinct MI355X (gfx950).

    from exact_attention_121_amd import attn_fwd, attn_bwd, attn_decode
    o, lse = attn_fwd(q, k, v, causal=True)     # torch fp16 tensors on the GPU
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=True)
    o1, lse1 = attn_decode(q_new, k_cache, v_cache)
    o = flash_attention(q, k, v, causal=True)   # differentiable (attn_fwd / attn_bwd)

The computation runs in hand-written HIP kernels behind a C ABI
(include/attn_fwd.h, libattn_fwd.so); this package is the thin binding,
the in-tree build script and the seeded input generator.
"""

from .binding import (  # noqa: F401
    ATTN_ERR_DEVICE,
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_SCRATCH,
    ATTN_ERR_UNSUPPORTED,
    ATTN_OK,
    BWD_NOALLOC_SCRATCH_BYTES,
    EXPORTS,
    AttnArgumentError,
    AttnError,
    AttnUnsupportedError,
    attn_bwd,
    attn_bwd_noalloc,
    attn_bwd_workspace_size,
    attn_check_args,
    attn_check_bwd_args,
    attn_check_decode_args,
    attn_decode,
    attn_decode_workspace_size,
    attn_fwd,
    attn_status_string,
    attn_version,
    load_library,
)
from .autograd import flash_attention, scaled_dot_product_attention  # noqa: F401

__version__ = "0.4.0"
