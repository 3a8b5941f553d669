"""GPU parity of the bf16 forward (attn_fwd_bf16) against the fp64 oracle.

Inputs are the fp16 workloads' draws rounded to bfloat16; the oracle widens
those bf16 values exactly.  Bar (bf16's unit roundoff is 2^-8, eight times
fp16's): P is rounded to bf16 for P.V and l sums those rounded values, so
the weights of the average move by at most 2^-8 relative and LSE by at most
2^-8 (3.9e-3); O is rounded to bf16 (2^-8 relative).  Hence
    max |O_gpu - O_ref| <= 4e-2,  mean |O_gpu - O_ref| <= 4e-3,
    max |LSE_gpu - LSE_ref| <= 4e-3, no NaN/Inf.
"""

import sys

import numpy as np
import pytest

from exact_attention_121_amd.inputs import WORKLOADS, make_qkv_bf16, sample_rows
from oracle.attention import attention_ref
from parity_util import assert_parity, convex_hull_ok, gather_rows

pytestmark = pytest.mark.gpu

BF16_MAX_O, BF16_MEAN_O, BF16_LSE = 4e-2, 4e-3, 4e-3


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def gpu_attention_bf16(q, k, v, scale, causal):
    import torch

    import exact_attention_121_amd as ea
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(torch.bfloat16) for x in (q, k, v))
    o, lse = ea.attn_fwd(tq, tk, tv, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(o, lse, O_ref, L_ref, what):
    mx, mean = assert_parity(o, lse, O_ref, L_ref, what=what, max_abs=BF16_MAX_O, mean_abs=BF16_MEAN_O,
                             lse_abs=BF16_LSE)
    _say(f"[bf16] {what}: max|dO| {mx:.2e} mean|dO| {mean:.2e}")


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_named_workload_bf16(wid):
    w = WORKLOADS[wid]
    _say(f"[bf16] workload {wid} {w.name}: {w.describe()}")
    q, k, v = make_qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, w.sigma, w.spike_frac, w.spike_mult)
    o, lse = gpu_attention_bf16(q, k, v, w.scale, w.causal)
    assert convex_hull_ok(o, v, w.Hq, slack=8e-3), "an output row left the value range"
    if wid in (1, 2):
        O_ref, L_ref = attention_ref(q, k, v, w.scale, causal=w.causal)
        check(o, lse, O_ref, L_ref, w.name)
    else:
        rows = sample_rows(w, count=256)
        O_ref, L_ref = attention_ref(q, k, v, w.scale, causal=w.causal, rows=rows)
        check(gather_rows(o, rows), gather_rows(lse[..., None], rows)[..., 0], O_ref, L_ref, w.name)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 129, 1000])
def test_edges_bf16(N, causal, d):
    Hq, Hkv = (8, 2) if N % 2 else (4, 4)
    _say(f"[bf16] edge N={N} d={d} causal={causal}")
    q, k, v = make_qkv_bf16(2, Hq, Hkv, N, d, seed=700 + N + d)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = gpu_attention_bf16(q, k, v, scale, causal)
    O_ref, L_ref = attention_ref(q, k, v, scale, causal=causal)
    check(o, lse, O_ref, L_ref, f"edge N={N} d={d} causal={causal}")


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_other_scales_bf16(scale):
    q, k, v = make_qkv_bf16(1, 4, 2, 300, 128, seed=77)
    for causal in (False, True):
        o, lse = gpu_attention_bf16(q, k, v, scale, causal)
        O_ref, L_ref = attention_ref(q, k, v, scale, causal=causal)
        check(o, lse, O_ref, L_ref, f"scale={scale} causal={causal}")


# --- backward and decode in bf16 -------------------------------------------

# Backward bar, per gradient X: max |dX| <= 4e-2 max |X_ref|, mean |dX| <=
# 8e-3 mean |X_ref| (the fp16 bar scaled by 4 of the 8x coarser unit
# roundoff: P, dS and the gradients are each rounded to bf16 once); where
# X_ref is identically 0, |X_gpu| <= 1e-4.
BF16_BWD_MAX_REL, BF16_BWD_MEAN_REL, BF16_BWD_ZERO = 4e-2, 8e-3, 1e-4


def _bf16_dout(shape, seed):
    from exact_attention_121_amd.inputs import round_to_bf16
    return round_to_bf16(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


def gpu_backward_bf16(q, k, v, do, scale, causal):
    import torch

    import exact_attention_121_amd as ea
    tq, tk, tv, tdo = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(torch.bfloat16)
                       for x in (q, k, v, do))
    o, lse = ea.attn_fwd(tq, tk, tv, scale=scale, causal=causal)
    grads = ea.attn_bwd(tq, tk, tv, o, lse, tdo, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert all(g.dtype == torch.bfloat16 for g in grads)
    return [g.float().cpu().numpy() for g in grads]


def check_grads(got, ref, what):
    stats = []
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        x = np.asarray(x, dtype=np.float64)
        assert np.isfinite(x).all(), f"{what} {name}: non-finite"
        err = np.abs(x - r)
        rmax, rmean = float(np.abs(r).max()), float(np.abs(r).mean())
        stats.append(f"{name} {err.max():.2e}/{rmax:.2e} mean {err.mean():.2e}/{rmean:.2e}")
        if rmax == 0.0:
            assert err.max() <= BF16_BWD_ZERO, f"{what} {name}: expected zeros, max {err.max():.3e}"
            continue
        assert err.max() <= BF16_BWD_MAX_REL * rmax, f"{what} {name}: max {err.max():.3e} vs {rmax:.3e}"
        assert err.mean() <= BF16_BWD_MEAN_REL * rmean, f"{what} {name}: mean {err.mean():.3e} vs {rmean:.3e}"
    _say(f"[bf16 bwd] {what}: " + "; ".join(stats))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (2, 4, 2, 63), (1, 2, 1, 129), (1, 4, 1, 777)])
def test_backward_bf16(shape, causal, d):
    from oracle.backward import attention_bwd_ref
    B, Hq, Hkv, N = shape
    q, k, v = make_qkv_bf16(B, Hq, Hkv, N, d, seed=800 + N + d)
    do = _bf16_dout(q.shape, 1800 + N + d)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    got = gpu_backward_bf16(q, k, v, do, scale, causal)
    check_grads(got, attention_bwd_ref(q, k, v, do, scale, causal=causal), f"{shape} d={d} causal={causal}")


def test_backward_bf16_llama7b_layer():
    """The LLaMA-7B layer shape at full size; the oracle checks two heads."""
    from oracle.backward import attention_bwd_ref
    w = WORKLOADS[2]
    q, k, v = make_qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    do = _bf16_dout(q.shape, w.seed + 7)
    got = gpu_backward_bf16(q, k, v, do, w.scale, w.causal)
    for b, h in ((0, 0), (1, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = attention_bwd_ref(q[sl], k[sl], v[sl], do[sl], w.scale, causal=w.causal)
        check_grads([x[sl] for x in got], ref, f"llama7b_layer head ({b}, {h})")


@pytest.mark.parametrize("shape", [(2, 8, 2, 1, 3000), (1, 32, 1, 16, 2100), (64, 8, 8, 1, 200), (1, 4, 4, 5, 5)])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_bf16(shape, d):
    import torch

    import exact_attention_121_amd as ea
    from oracle.attention import attention_decode_ref
    B, Hq, Hkv, Nq, Nk = shape
    rng_seed = 900 + Nk + d
    q = make_qkv_bf16(B, Hq, Hkv, Nq, d, seed=rng_seed)[0]
    _, k, v = make_qkv_bf16(B, Hkv, Hkv, Nk, d, seed=rng_seed + 1)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(torch.bfloat16) for x in (q, k, v))
    for causal in (True, False):
        o, lse = ea.attn_decode(tq, tk, tv, scale=float(np.float32(1 / np.sqrt(d))), causal=causal)
        torch.cuda.synchronize()
        O_ref, L_ref = attention_decode_ref(q, k, v, float(np.float32(1 / np.sqrt(d))), causal=causal)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref, f"decode {shape} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 96, 160, 224])
def test_backward_bf16_subtile_form(d):
    """bf16 gradients from the sub-tile form of the dK/dV kernel (non-causal,
    a grid of 512 dK/dV workgroups: B=4, H=16, N=1000); the oracle checks two
    whole heads."""
    from oracle.backward import attention_bwd_ref
    B, H, N = 4, 16, 1000
    _say(f"[bf16 bwd] sub-tile form B={B} H={H} N={N} d={d}")
    q, k, v = make_qkv_bf16(B, H, H, N, d, seed=2300 + d)
    do = _bf16_dout(q.shape, 2400 + d)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    got = gpu_backward_bf16(q, k, v, do, scale, False)
    for b, h in ((0, 0), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = attention_bwd_ref(q[sl], k[sl], v[sl], do[sl], scale, causal=False)
        check_grads([x[sl] for x in got], ref, f"sub-tile form d={d} head ({b}, {h})")
