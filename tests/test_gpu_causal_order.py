"""GPU parity on causal shapes whose work order interleaves several heads.

With the causal mask the forward, dQ and dK/dV kernels run the tiles of a
group of heads heaviest first (the group size is chosen on the host from the
grid, the tiles per head and the bytes each head streams).  The named
workloads exercise groups of 4 and 8 heads on sampled rows; these shapes are
small enough for the oracle to check every row and every gradient, and each
gives a group of at least two heads in the kernel named next to it (grid of
8 x per-XCD heads x tiles per head):

  * B=1, H=16, N=1024, d=128: forward and dQ groups of 2 (128 query tiles,
    2 heads per XCD), dK/dV groups of 2 (128 key tiles);
  * B=2, Hq=8, Hkv=2, N=512, d=64 (GQA): forward and dQ groups of 2;
  * B=1, H=32, N=2048, d=64: groups of 4 (heads of 512 KB of K/V).

A wrong order (a tile computed twice and another never) fails parity.
"""

import sys

import numpy as np
import pytest

from exact_attention_121_amd.inputs import make_qkv
from oracle.attention import attention_ref
from oracle.backward import attention_bwd_ref
from parity_util import assert_parity, gpu_attention
from test_gpu_backward import assert_grad_parity, gpu_backward, make_dout

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16, 16, 1024, 128), (2, 8, 2, 512, 64), (1, 32, 32, 2048, 64)]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("B,Hq,Hkv,N,d", SHAPES)
def test_forward_grouped_causal(B, Hq, Hkv, N, d):
    _say(f"[causal order] forward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=7100 + N + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_attention(q, k, v, scale, True)
    O_ref, L_ref = attention_ref(q, k, v, np.float32(scale), causal=True)
    assert_parity(o, lse, O_ref, L_ref, what=f"grouped causal B={B} Hq={Hq} N={N} d={d}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d", SHAPES[:2])
def test_backward_grouped_causal(B, Hq, Hkv, N, d):
    _say(f"[causal order] backward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=7200 + N + d)
    do = make_dout(q.shape, seed=7300 + N + d)
    scale = 1.0 / np.sqrt(d)
    got = gpu_backward(q, k, v, do, scale, True)
    ref = attention_bwd_ref(q, k, v, do, np.float32(scale), causal=True)
    assert_grad_parity(got, ref, f"grouped causal backward B={B} Hq={Hq} N={N} d={d}")
