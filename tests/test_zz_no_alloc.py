"""attn_bwd_noalloc, the allocation-free backward, through the C ABI.

It runs the same kernels as attn_bwd with the per-row terms in the library's
fixed scratch array instead of a caller workspace.  Two calls in a row, the
second on a smaller problem (so that it sees the scratch as the first call
left it), must give exactly attn_bwd's gradients, which are held to the fp64
oracle's bar here as well; a problem beyond the scratch is refused on the
host with ATTN_ERR_SCRATCH.
"""

import sys

import numpy as np
import pytest

import exact_attention_121_amd as ea
from exact_attention_121_amd.inputs import make_qkv
from oracle.backward import attention_bwd_ref
from parity_util import to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(B, Hq, Hkv, N, d, causal, seed):
    import torch

    qn, kn, vn = make_qkv(B, Hq, Hkv, N, d, seed=seed)
    don = np.random.default_rng(seed + 1).standard_normal(qn.shape, dtype=np.float32).astype(np.float16)
    q, k, v, do = to_dev(qn, kn, vn, don)
    o, lse = ea.attn_fwd(q, k, v, causal=causal)
    want = ea.attn_bwd(q, k, v, o, lse, do, causal=causal)
    got = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan")))
    ea.attn_bwd_noalloc(q, k, v, o, lse, do, *got, causal=causal)
    torch.cuda.synchronize()
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        assert torch.equal(g, w), f"{name}: attn_bwd_noalloc differs from attn_bwd"
    scale = float(np.float32(1.0 / np.sqrt(d)))
    refs = attention_bwd_ref(qn, kn, vn, don, scale, causal=causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, refs):
        err = np.abs(g.cpu().numpy().astype(np.float64) - r)
        assert np.isfinite(err).all(), name
        assert err.max() <= 1e-2 * np.abs(r).max() and err.mean() <= 2e-3 * np.abs(r).mean(), name


def test_two_calls_second_smaller():
    _say("[noalloc] B=2 Hq=8 Hkv=2 N=1000 d=128 causal, then B=1 Hq=4 Hkv=4 N=300 d=64")
    _case(2, 8, 2, 1000, 128, True, seed=811)
    _case(1, 4, 4, 300, 64, False, seed=812)


def test_largest_problem_and_the_limit():
    import torch

    # 2^21 padded rows exactly: B=1, Hq=64, N=32768 (d=32 keeps it quick).
    B, Hq, N, d = 1, 64, 32768, 32
    assert ea.attn_bwd_workspace_size(B, Hq, N, d) == ea.BWD_NOALLOC_SCRATCH_BYTES
    _say(f"[noalloc] at the scratch limit: B={B} Hq={Hq} N={N} d={d}")
    q, k, v = to_dev(*make_qkv(B, Hq, 8, N, d, seed=813))
    do = torch.randn_like(q)
    o, lse = ea.attn_fwd(q, k, v)
    want = ea.attn_bwd(q, k, v, o, lse, do)
    got = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ea.attn_bwd_noalloc(q, k, v, o, lse, do, *got)
    torch.cuda.synchronize()
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        assert torch.equal(g, w), name
    # One more query tile per head is over the limit: refused, nothing written.
    q2 = torch.zeros(B, Hq, N + 1, d, dtype=torch.float16, device=q.device)
    k2 = torch.zeros(B, 8, N + 1, d, dtype=torch.float16, device=q.device)
    l2 = torch.zeros(B, Hq, N + 1, dtype=torch.float32, device=q.device)
    outs = (torch.ones_like(q2), torch.ones_like(k2), torch.ones_like(k2))
    with pytest.raises(ea.AttnError) as e:
        ea.attn_bwd_noalloc(q2, k2, k2.clone(), q2.clone(), l2, q2.clone(), *outs)
    assert e.value.status == ea.ATTN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert all(bool((t == 1).all()) for t in outs)
