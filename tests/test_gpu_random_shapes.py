"""Seeded random shapes against the fp64 oracle (forward and backward, fp16).

Forty problems drawn from one fixed seed: batch 1-3, 1-8 query heads with a
random divisor as K/V heads (GQA and MQA included), sequence lengths from 1 to
1 500 (ragged against every tile size), every supported head_dim, causal or
not, a random scale (negative and zero included) and, for some, 1 % of Q and K
rows multiplied by 8.  Each is compared with the oracle at the parity bar.
Sixteen backward problems are drawn the same way (shorter sequences; scales
1, 0.5, -1 and 0 over sqrt(d)) and held to the backward bar.  The draws are
fixed, so a failure names a reproducible problem.
"""

import numpy as np
import pytest

from exact_attention_121_amd.inputs import make_qkv
from oracle.attention import attention_ref
from parity_util import assert_parity, gpu_attention

pytestmark = pytest.mark.gpu


def _problems(count=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        B = int(rng.integers(1, 4))
        Hq = int(rng.integers(1, 9))
        divisors = [h for h in range(1, Hq + 1) if Hq % h == 0]
        Hkv = int(rng.choice(divisors))
        N = int(rng.choice([1, 2, 31, 33, 63, 65, 127, 129, 255, 257, 300, 511, 777, 1000, 1500]))
        d = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256]))
        causal = bool(rng.integers(0, 2))
        kind = int(rng.integers(0, 6))
        scale = {0: 1.0 / np.sqrt(d), 1: 0.5 / np.sqrt(d), 2: 2.0 / np.sqrt(d), 3: -1.0 / np.sqrt(d), 4: 0.0,
                 5: 1.0 / np.sqrt(d)}[kind]
        spikes = 0.01 if kind == 5 else 0.0
        out.append((i, B, Hq, Hkv, N, d, causal, float(np.float32(scale)), spikes))
    return out


@pytest.mark.parametrize("prob", _problems(), ids=lambda p: f"p{p[0]}")
def test_random_shape(prob):
    i, B, Hq, Hkv, N, d, causal, scale, spikes = prob
    print(f"[random] {prob}", flush=True)
    qn, kn, vn = make_qkv(B, Hq, Hkv, N, d, seed=9000 + i, spike_frac=spikes, spike_mult=8.0)
    O_ref, L_ref = attention_ref(qn, kn, vn, scale, causal=causal)
    o, lse = gpu_attention(qn, kn, vn, scale, causal)
    assert_parity(o, lse, O_ref, L_ref, what=f"random {prob}")


def _bwd_problems(count=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        B = int(rng.integers(1, 3))
        Hq = int(rng.integers(1, 7))
        Hkv = int(rng.choice([h for h in range(1, Hq + 1) if Hq % h == 0]))
        N = int(rng.choice([1, 17, 64, 100, 129, 300, 513, 700]))
        d = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256]))
        causal = bool(rng.integers(0, 2))
        scale = float(np.float32(rng.choice([1.0, 0.5, -1.0, 0.0]) / np.sqrt(d)))
        out.append((i, B, Hq, Hkv, N, d, causal, scale))
    return out


@pytest.mark.parametrize("prob", _bwd_problems(), ids=lambda p: f"b{p[0]}")
def test_random_shape_backward(prob):
    from oracle.backward import attention_bwd_ref
    from test_gpu_backward import assert_grad_parity, gpu_backward, make_dout

    i, B, Hq, Hkv, N, d, causal, scale = prob
    print(f"[random bwd] {prob}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=9500 + i)
    do = make_dout(q.shape, seed=9700 + i)
    got = gpu_backward(q, k, v, do, scale, causal)
    ref = attention_bwd_ref(q, k, v, do, scale, causal=causal)
    assert_grad_parity(got, ref, f"random bwd {prob}")
