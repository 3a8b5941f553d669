"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

    from exact_attention_121_amd import attn_fwd
    o, lse = attn_fwd(q, k, v, causal=True)     # torch fp16 tensors on the GPU

The computation runs in hand-written HIP kernels behind a C ABI
(include/attn_fwd.h, libattn_fwd.so); this package is the thin binding,
the in-tree build script and the seeded input generator.
"""

from .binding import (  # noqa: F401
    ATTN_ERR_DEVICE,
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_UNSUPPORTED,
    ATTN_OK,
    EXPORTS,
    AttnArgumentError,
    AttnError,
    AttnUnsupportedError,
    attn_check_args,
    attn_check_decode_args,
    attn_decode,
    attn_decode_workspace_size,
    attn_fwd,
    attn_status_string,
    attn_version,
    load_library,
)

__version__ = "0.2.0"
