"""GPU tests of the library's compile-time variants (exact_attention_121_amd/build.py).

* Race check: the ``paranoid`` build waits for every copy and LDS access and
  puts a workgroup barrier at each phase boundary of the pipelined loops, with
  the same arithmetic in the same order.  On the five workloads' shapes
  (scaled down to a few heads) and on ragged sizes, its forward, decode and
  backward outputs must equal the default build's bit for bit: a stage read
  before its copy landed, or refilled while a wave still read it, would show
  as a difference.
* Tile variants: the ``bn32`` build (the offline sweep's runner-up tiles:
  32-key tiles at head_dim 128, one query block per wave with 64-key tiles
  at head_dim 64) and the ``pp`` build (the 8-wave ping-pong kernel for the
  head_dim 128 non-causal forward) are held to the fp64 oracle, like the
  default build.
"""

import functools
import os
import sys

import numpy as np
import pytest

import exact_attention_121_amd as ea
from exact_attention_121_amd.build import variant_path
from exact_attention_121_amd.inputs import make_decode_qkv, make_qkv
from oracle.attention import attention_ref
from parity_util import assert_parity, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def _variant(name):
    path = variant_path(name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the library with its variants (__graft_entry__.build())")
    return ea.load_library(path)


# (B, Hq, Hkv, N, d, causal, sigma, spike_frac): the five workloads with
# fewer heads and batch entries, then ragged sizes.
RACE_SHAPES = [
    (1, 1, 1, 128, 64, False, 1.0, 0.0),
    (1, 4, 4, 2048, 128, False, 1.0, 0.0),
    (1, 4, 4, 4096, 64, True, 1.0, 0.01),
    (1, 8, 2, 2048, 256, True, 1.0, 0.0),
    (1, 4, 1, 8192, 128, True, 0.5, 0.0),
    (2, 4, 2, 1000, 96, True, 1.0, 0.0),
    (1, 2, 1, 333, 160, False, 1.0, 0.0),
]


@pytest.mark.parametrize("shape", RACE_SHAPES)
def test_paranoid_build_forward_is_bitwise_equal(shape):
    import torch

    B, Hq, Hkv, N, d, causal, sigma, spikes = shape
    _say(f"[race] forward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = to_dev(*make_qkv(B, Hq, Hkv, N, d, seed=300 + N + d, sigma=sigma, spike_frac=spikes,
                               spike_mult=8.0))
    o0, l0 = ea.attn_fwd(q, k, v, causal=causal)
    o1, l1 = ea.attn_fwd(q, k, v, causal=causal, library=_variant("paranoid"))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("shape", [(4, 32, 8, 1, 8192, 128), (1, 32, 1, 1, 40000, 128), (2, 16, 4, 5, 3000, 256)])
def test_paranoid_build_decode_is_bitwise_equal(shape):
    import torch

    _say(f"[race] decode {shape}")
    q, k, v = to_dev(*make_decode_qkv(*shape, seed=400 + shape[4]))
    o0, l0 = ea.attn_decode(q, k, v, causal=True)
    o1, l1 = ea.attn_decode(q, k, v, causal=True, library=_variant("paranoid"))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("shape", [(1, 4, 4, 2048, 128, False), (1, 4, 4, 1000, 64, True),
                                   (1, 8, 2, 700, 256, True), (4, 16, 16, 1000, 128, False)])
def test_paranoid_build_backward_is_bitwise_equal(shape):
    import torch

    B, Hq, Hkv, N, d, causal = shape
    _say(f"[race] backward B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = to_dev(*make_qkv(B, Hq, Hkv, N, d, seed=500 + N + d))
    do = torch.randn_like(q)
    o, lse = ea.attn_fwd(q, k, v, causal=causal)
    g0 = ea.attn_bwd(q, k, v, o, lse, do, causal=causal)
    g1 = ea.attn_bwd(q, k, v, o, lse, do, causal=causal, library=_variant("paranoid"))
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), g0, g1):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("shape", [(1, 2, 2, 2048, 128, False), (1, 4, 2, 1000, 64, True),
                                   (2, 2, 1, 777, 128, True), (1, 1, 1, 4096, 64, True)])
def test_bn32_variant_against_the_oracle(shape):
    import torch

    B, Hq, Hkv, N, d, causal = shape
    _say(f"[variant bn32] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    qn, kn, vn = make_qkv(B, Hq, Hkv, N, d, seed=600 + N + d, spike_frac=0.01, spike_mult=8.0)
    q, k, v = to_dev(qn, kn, vn)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = ea.attn_fwd(q, k, v, scale=scale, causal=causal, library=_variant("bn32"))
    torch.cuda.synchronize()
    O_ref, L_ref = attention_ref(qn, kn, vn, scale, causal=causal)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref, what=f"bn32 {shape}")


@pytest.mark.parametrize("shape", [(1, 2, 2, 2048, 128, False), (2, 3, 1, 777, 128, False), (1, 1, 1, 33, 128, False),
                                   (1, 4, 2, 1000, 128, False)])
def test_pp_variant_against_the_oracle(shape):
    import torch

    B, Hq, Hkv, N, d, causal = shape
    _say(f"[variant pp] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    qn, kn, vn = make_qkv(B, Hq, Hkv, N, d, seed=700 + N, spike_frac=0.01, spike_mult=8.0)
    q, k, v = to_dev(qn, kn, vn)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = ea.attn_fwd(q, k, v, scale=scale, causal=causal, library=_variant("pp"))
    torch.cuda.synchronize()
    O_ref, L_ref = attention_ref(qn, kn, vn, scale, causal=causal)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref, what=f"pp {shape}")
