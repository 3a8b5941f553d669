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
