"""GPU parity at the head_dims beyond 64, 128 and 256: 32, 96, 160, 192, 224.

The pages' fused operator takes head_dim 64, 128 or 256 and falls back to
unfused attention otherwise ([CANN-FA], the closing note on head_dim); this
library runs its fused kernels for every multiple of 32 up to 256, padding
the LDS tile rows to 8, 16 or 32 chunks.  These tests hold those kernels to
the same oracle and the same bars as the other head_dims:

* forward and decode, fp16: max |dO| <= 1e-2, mean |dO| <= 1e-3,
  max |dLSE| <= 1e-3;
* forward and decode, bf16: 4e-2 / 4e-3 / 4e-3 (bf16's unit roundoff is
  2^-8, eight times fp16's);
* backward, fp16: per gradient, max error <= 1e-2 * max |ref| and mean error
  <= 2e-3 * mean |ref|; bf16: 4e-2 and 8e-3.
"""

import sys

import numpy as np
import pytest

from exact_attention_121_amd.inputs import make_decode_qkv, make_qkv, make_qkv_bf16
from oracle.attention import attention_decode_ref, attention_ref
from oracle.backward import attention_bwd_ref
from parity_util import assert_parity, convex_hull_ok, gather_rows, gpu_attention
from test_gpu_backward import assert_grad_parity, gpu_backward, make_dout
from test_gpu_bf16 import _bf16_dout, check, check_grads, gpu_attention_bf16, gpu_backward_bf16
from test_gpu_decode import gpu_decode

pytestmark = pytest.mark.gpu

NEW_DIMS = [32, 96, 160, 192, 224]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _scale(d):
    return float(np.float32(1.0 / np.sqrt(d)))


# (B, Hq, Hkv, N): one key, ragged tails around the 32 / 64 / 128 tile sizes,
# GQA and MQA groupings.
FWD_EDGE = [(1, 1, 1, 1), (2, 2, 1, 7), (1, 4, 2, 65), (2, 4, 4, 129), (1, 8, 2, 300), (1, 6, 1, 1000)]


@pytest.mark.parametrize("d", NEW_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FWD_EDGE)
def test_forward_new_dims(shape, causal, d):
    B, Hq, Hkv, N = shape
    _say(f"[hd] forward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=1100 + N + d)
    o, lse = gpu_attention(q, k, v, _scale(d), causal)
    O_ref, L_ref = attention_ref(q, k, v, _scale(d), causal=causal)
    assert_parity(o, lse, O_ref, L_ref, what=f"forward {shape} d={d} causal={causal}")


@pytest.mark.parametrize("d", NEW_DIMS)
def test_forward_new_dims_long(d):
    """N = 4096 (causal, GQA 8:2): many key tiles per workgroup; the oracle
    checks 48 sampled rows per head (both ends included), the value range
    holds everywhere."""
    B, Hq, Hkv, N = 1, 8, 2, 4096
    _say(f"[hd] forward long N={N} d={d}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=1200 + d)
    o, lse = gpu_attention(q, k, v, _scale(d), True)
    assert convex_hull_ok(o, v, Hq), "an output row left the value range"
    rng = np.random.default_rng(1300 + d)
    rows = np.sort(np.stack([np.stack([np.concatenate([[0, N - 1], rng.choice(np.arange(1, N - 1), 46, replace=False)])
                                       for _ in range(Hq)]) for _ in range(B)]), axis=-1)
    O_ref, L_ref = attention_ref(q, k, v, _scale(d), causal=True, rows=rows)
    mx, mean = assert_parity(gather_rows(o, rows), gather_rows(lse[..., None], rows)[..., 0], O_ref, L_ref,
                             what=f"forward long d={d}")
    _say(f"[hd] forward long d={d}: max|dO| {mx:.2e} mean|dO| {mean:.2e}")


@pytest.mark.parametrize("d", NEW_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [63, 1000])
def test_forward_new_dims_bf16(N, causal, d):
    _say(f"[hd] forward bf16 N={N} d={d} causal={causal}")
    q, k, v = make_qkv_bf16(2, 4, 2, N, d, seed=1400 + N + d)
    o, lse = gpu_attention_bf16(q, k, v, _scale(d), causal)
    O_ref, L_ref = attention_ref(q, k, v, _scale(d), causal=causal)
    check(o, lse, O_ref, L_ref, f"forward bf16 N={N} d={d} causal={causal}")


# (B, Hq, Hkv, Nq, Nk): one key; packed rows 24 with a ragged key tile; two
# row blocks; many splits (merge over 32-dim slices); one split (no merge).
DEC_EDGE = [(1, 1, 1, 1, 1), (1, 8, 1, 3, 129), (3, 8, 2, 16, 1000), (1, 2, 1, 1, 4097), (64, 8, 8, 1, 200)]


@pytest.mark.parametrize("d", NEW_DIMS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", DEC_EDGE)
def test_decode_new_dims(shape, causal, d):
    B, Hq, Hkv, Nq, Nk = shape
    _say(f"[hd] decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    q, k, v = make_decode_qkv(B, Hq, Hkv, Nq, Nk, d, seed=1500 + Nk + d + Nq)
    o, lse = gpu_decode(q, k, v, _scale(d), causal)
    O_ref, L_ref = attention_decode_ref(q, k, v, _scale(d), causal=causal)
    assert_parity(o, lse, O_ref, L_ref, what=f"decode {shape} d={d} causal={causal}")


@pytest.mark.parametrize("d", NEW_DIMS)
def test_decode_new_dims_bf16(d):
    import torch

    import exact_attention_121_amd as ea
    B, Hq, Hkv, Nq, Nk = 2, 8, 2, 1, 3000
    _say(f"[hd] decode bf16 d={d}")
    q = make_qkv_bf16(B, Hq, Hkv, Nq, d, seed=1600 + d)[0]
    _, k, v = make_qkv_bf16(B, Hkv, Hkv, Nk, d, seed=1601 + d)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(torch.bfloat16) for x in (q, k, v))
    for causal in (True, False):
        o, lse = ea.attn_decode(tq, tk, tv, scale=_scale(d), causal=causal)
        torch.cuda.synchronize()
        O_ref, L_ref = attention_decode_ref(q, k, v, _scale(d), causal=causal)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref, f"decode bf16 d={d} causal={causal}")


BWD_EDGE = [(1, 1, 1, 1), (2, 4, 2, 63), (1, 2, 1, 129), (2, 8, 2, 300), (1, 4, 1, 777)]


@pytest.mark.parametrize("d", NEW_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", BWD_EDGE)
def test_backward_new_dims(shape, causal, d):
    B, Hq, Hkv, N = shape
    _say(f"[hd] backward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=1700 + N + d)
    do = make_dout(q.shape, seed=1800 + N + d)
    got = gpu_backward(q, k, v, do, _scale(d), causal)
    ref = attention_bwd_ref(q, k, v, do, _scale(d), causal=causal)
    assert_grad_parity(got, ref, f"backward {shape} d={d} causal={causal}")


@pytest.mark.parametrize("d", NEW_DIMS)
def test_backward_new_dims_bf16(d):
    B, Hq, Hkv, N = 1, 4, 2, 300
    _say(f"[hd] backward bf16 d={d}")
    q, k, v = make_qkv_bf16(B, Hq, Hkv, N, d, seed=1900 + d)
    do = _bf16_dout(q.shape, 1950 + d)
    for causal in (False, True):
        got = gpu_backward_bf16(q, k, v, do, _scale(d), causal)
        check_grads(got, attention_bwd_ref(q, k, v, do, _scale(d), causal=causal), f"bf16 d={d} causal={causal}")
