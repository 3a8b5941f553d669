"""Closed-form pins and robustness checks of the HIP path on the GPU.

Each pin is a fact of the softmax definition that the kernel must meet on
its own (not only agreement with the oracle): causal row 0 copies v_0
bit for bit, scale 0 gives prefix means and LSE = ln(count) even at
N = 131072 (which needs an fp32 running sum), GQA equals repeated K/V heads
bit for bit, and P's rows sum to 1.  Robustness: untouched guard bands,
bitwise determinism, non-default streams, the lse=NULL path and empty
problems.
"""

import math
import sys

import numpy as np
import pytest

import exact_attention_121_amd as ea
from exact_attention_121_amd.inputs import make_qkv
from oracle.attention import attention_ref
from parity_util import assert_parity, gpu_attention, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_causal_row0_copies_v0(d):
    _say(f"[pin] causal row 0, d={d}")
    q, k, v = make_qkv(2, 4, 2, 200, d, seed=1)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = gpu_attention(q, k, v, scale, True)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, h, 0], v[b, h // 2, 0]), f"b={b} h={h}"
            s00 = float(np.float32(scale)) * float(q[b, h, 0].astype(np.float64) @ k[b, h // 2, 0].astype(np.float64))
            assert abs(lse[b, h, 0] - s00) <= 1e-3


@pytest.mark.parametrize("N,d", [(1000, 64), (4097, 128), (131072, 64)])
def test_scale_zero_prefix_means(N, d):
    _say(f"[pin] scale 0, N={N} d={d}")
    q, k, v = make_qkv(1, 1, 1, N, d, seed=2)
    o, lse = gpu_attention(q, k, v, 0.0, True)
    counts = np.arange(1, N + 1, dtype=np.float64)
    prefix_mean = np.cumsum(v[0, 0].astype(np.float64), axis=0) / counts[:, None]
    err = np.abs(o[0, 0].astype(np.float64) - prefix_mean)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())
    assert np.abs(lse[0, 0] - np.log(counts)).max() <= 1e-3
    if N == 131072:
        assert abs(lse[0, 0, -1] - math.log(131072)) <= 1e-3  # an fp16 running sum would overflow
    o2, lse2 = gpu_attention(q, k, v, 0.0, False)
    mean = v[0, 0].astype(np.float64).mean(axis=0)
    assert np.abs(o2[0, 0].astype(np.float64) - mean).max() <= 1e-2
    assert np.abs(lse2[0, 0] - math.log(N)).max() <= 1e-3


def test_gqa_equals_repeated_heads_bitwise():
    _say("[pin] GQA == repeated K/V heads")
    for Hq, Hkv in ((8, 2), (8, 1), (6, 3)):
        q, k, v = make_qkv(2, Hq, Hkv, 333, 128, seed=3)
        G = Hq // Hkv
        for causal in (False, True):
            o1, l1 = gpu_attention(q, k, v, 0.1, causal)
            o2, l2 = gpu_attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.1, causal)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rows_of_p_sum_to_one():
    """V = identity (N <= d): O = P, so each row sums to 1 within fp16 error."""
    _say("[pin] rows of P sum to 1")
    for d in (64, 128, 256):
        N = d
        q, k, _ = make_qkv(1, 2, 2, N, d, seed=4)
        v = np.broadcast_to(np.eye(N, d, dtype=np.float16), (1, 2, N, d)).copy()
        for causal in (False, True):
            o, _ = gpu_attention(q, k, v, float(np.float32(1 / math.sqrt(d))), causal)
            s = o.astype(np.float64).sum(axis=-1)
            assert np.abs(s - 1).max() <= 2e-3, np.abs(s - 1).max()
            assert (o >= 0).all()
            if causal:
                assert np.all(np.triu(o[0, 0].astype(np.float64), 1) == 0.0)


def test_constant_values_give_constant_output():
    _say("[pin] constant V")
    q, k, _ = make_qkv(1, 4, 4, 517, 128, seed=5)
    v = np.full((1, 4, 517, 128), 1.5, dtype=np.float16)
    for causal in (False, True):
        o, _ = gpu_attention(q, k, v, 0.09, causal)
        assert np.abs(o.astype(np.float64) - 1.5).max() <= 2e-3


def test_guard_bands_untouched():
    import torch
    _say("[robust] guard bands")
    B, Hq, Hkv, N, d = 2, 4, 2, 130, 128
    q, k, v = to_dev(*make_qkv(B, Hq, Hkv, N, d, seed=6))
    guard = 4096
    n_o = B * Hq * N * d
    obuf = torch.full((n_o + 2 * guard,), 7.0, dtype=torch.float16, device="cuda:0")
    lbuf = torch.full((B * Hq * N + 2 * guard,), -3.0, dtype=torch.float32, device="cuda:0")
    o = obuf[guard:guard + n_o].view(B, Hq, N, d)
    lse = lbuf[guard:guard + B * Hq * N].view(B, Hq, N)
    for causal in (False, True):
        ea.attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert (obuf[:guard] == 7.0).all() and (obuf[guard + n_o:] == 7.0).all()
        assert (lbuf[:guard] == -3.0).all() and (lbuf[guard + B * Hq * N:] == -3.0).all()
        O_ref, L_ref = attention_ref(*(x.cpu().numpy() for x in (q, k, v)), 1 / math.sqrt(d), causal=causal)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref, what="guarded")


def test_deterministic_streams_and_lse_optional():
    import torch
    _say("[robust] determinism, streams, lse=None")
    q, k, v = to_dev(*make_qkv(2, 8, 2, 1000, 128, seed=8))
    for causal in (False, True):
        ref_o, ref_l = ea.attn_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        for _ in range(2):
            o, l = ea.attn_fwd(q, k, v, causal=causal)
            torch.cuda.synchronize()
            assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            o, l = ea.attn_fwd(q, k, v, causal=causal)
        s.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
        o2, l2 = ea.attn_fwd(q, k, v, causal=causal, return_lse=False)
        torch.cuda.synchronize()
        assert l2 is None and torch.equal(o2, ref_o)


def test_empty_and_unsupported():
    import torch
    _say("[robust] empty problems and unsupported head_dim")
    for shape in ((0, 4, 16, 64), (2, 4, 0, 64)):
        q = torch.empty(shape, dtype=torch.float16, device="cuda:0")
        o, l = ea.attn_fwd(q, q, q)
        assert o.shape == q.shape and l.shape == shape[:3]
    q = torch.zeros(1, 1, 16, 80, dtype=torch.float16, device="cuda:0")
    with pytest.raises(ea.AttnUnsupportedError):
        ea.attn_fwd(q, q, q)
    q = torch.zeros(1, 3, 16, 64, dtype=torch.float16, device="cuda:0")
    k = torch.zeros(1, 2, 16, 64, dtype=torch.float16, device="cuda:0")
    with pytest.raises(ea.AttnArgumentError):
        ea.attn_fwd(q, k, k)
