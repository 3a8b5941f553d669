"""GPU edge cases at the boundary of the library's sizes: empty problems, and
one key/value head of exactly 2^30 elements (2 GiB), the largest the 32-bit
buffer offsets address (loads past the end of a head use a base of 2^31).

The forward at that size is minutes of work; the decode path streams the same
head through the same tile loads in milliseconds, so it carries the check.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def test_empty_problems_launch_nothing():
    import torch

    import exact_attention_121_amd as ea
    dev = "cuda:0"
    for shape_q, shape_kv in (((0, 4, 16, 64), (0, 2, 16, 64)), ((2, 4, 0, 128), (2, 2, 0, 128))):
        q = torch.empty(shape_q, dtype=torch.float16, device=dev)
        k = torch.empty(shape_kv, dtype=torch.float16, device=dev)
        o, lse = ea.attn_fwd(q, k, k, causal=True)
        assert o.shape == q.shape and lse.shape == shape_q[:3]
        dq, dk, dv = ea.attn_bwd(q, k, k, o, lse, q, causal=True)
        assert dq.shape == q.shape and dk.shape == k.shape
    q = torch.empty((1, 4, 0, 64), dtype=torch.float16, device=dev)
    k = torch.randn((1, 2, 10, 64), device=dev).half()
    o, lse = ea.attn_decode(q, k, k)
    assert o.shape == q.shape
    torch.cuda.synchronize()


@pytest.mark.parametrize("causal", [True, False])
def test_decode_at_the_largest_head(causal):
    """Nk * d = 2^30 (8 388 608 keys of 128 dims, 2 GiB per K and V head),
    two new queries of two query heads (GQA); checked against the oracle."""
    import torch

    import exact_attention_121_amd as ea
    from oracle.attention import attention_decode_ref
    Nk, d = (1 << 30) // 128, 128
    _say(f"[limits] decode Nk={Nk} d={d} causal={causal}")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(4242)
    k = torch.randn((1, 1, Nk, d), device="cuda:0", generator=g).half()
    v = torch.randn((1, 1, Nk, d), device="cuda:0", generator=g).half()
    q = torch.randn((1, 2, 2, d), device="cuda:0", generator=g).half()
    o, lse = ea.attn_decode(q, k, v, scale=0.0884, causal=causal)
    torch.cuda.synchronize()
    q_np, k_np, v_np = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    del k, v
    O_ref, L_ref = attention_decode_ref(q_np, k_np, v_np, 0.0884, causal=causal)
    err = np.abs(o.cpu().numpy().astype(np.float64) - O_ref)
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - L_ref)
    _say(f"[limits] max|dO| {err.max():.2e} max|dLSE| {lerr.max():.2e}")
    assert np.isfinite(err).all() and err.max() <= 1e-2 and err.mean() <= 1e-3 and lerr.max() <= 1e-3
