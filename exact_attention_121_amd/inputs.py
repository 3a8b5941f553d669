"""Seeded synthetic inputs for the attention forward (shared by tests and bench).

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the GPU path's tests and the CPU oracle's callers
take their inputs from here.

Recipe (every draw uses numpy's PCG64 ``default_rng``):
  * Q, then K, then V are drawn in that order.  Each tensor is drawn one
    (b, h) head at a time, in (b, h) order, as ``standard_normal((N, d),
    dtype=float32) * sigma`` and cast to fp16 with round-to-nearest-even.
  * Spiky rows (the causal-prefill workload): right after a tensor's values
    are drawn (Q and K only), exactly round(frac * B * H * N) of its rows are
    chosen uniformly without replacement from the flattened (b, h, n) index
    and multiplied by ``spike_mult`` in fp32 before the fp16 cast.
  * Sampled query rows (the long-context workload): for head (b, hq) the rows
    are {0, N-1} plus R-2 distinct rows drawn uniformly without replacement
    from 1..N-2 by ``default_rng(seed + 10**6 + b*Hq + hq)``, sorted.

  * bf16 inputs: the same draws, rounded to bfloat16 (to nearest even)
    instead of fp16.
  * Decode inputs: Q [B, Hq, Nq, d] is drawn first, then K and V
    [B, Hkv, Nk, d], each as above (one head at a time, N(0, sigma^2)).

The workloads mirror the shapes the pages measure or show: the LLaMA-7B layer
(seq 2048, 32 heads, head_dim 128, fp16) of the FlashAttention operator page
on www.mooersco.com (section on the gap to standard attention), its
(2, 32, 2048, 128) fp16 SDPA example, the 4096/8192 sequence lengths of the
hwcomputing.csdn.net tutorial's measurement table, and the GQA/MQA and
128K-context statements of the gitcode.csdn.net page (section 6).  There are
no model weights or activations here, so N(0, sigma^2) values stand in for
them at the same shapes.  The decode workloads put one (or a few) new
queries against a cache of those lengths and head layouts; the batched one
is sized so that its cache (2 GiB) is several times the chip's last-level
cache, so that it measures HBM.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    sigma: float = 1.0
    spike_frac: float = 0.0
    spike_mult: float = 1.0
    sample_rows: int = 0          # 0: the oracle checks every row
    seed: int = 0

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to the fp32 value the library receives."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def pairs(self) -> int:
        """Visible (query, key) pairs over all heads."""
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.Hq * per_head

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs: 2d for q.k plus 2d for p*v per visible pair."""
        return 4 * self.d * self.pairs

    def describe(self) -> str:
        mask = "causal" if self.causal else "non-causal"
        heads = f"H={self.Hq}" if self.Hq == self.Hkv else f"Hq={self.Hq} Hkv={self.Hkv}"
        return f"B={self.B} {heads} N={self.N} d={self.d} {mask}"


WORKLOADS = {
    1: Workload("tiny_single_head", 1, 1, 1, 128, 64, False, seed=1001),
    2: Workload("llama7b_layer", 2, 32, 32, 2048, 128, False, seed=1002),
    3: Workload("causal_prefill_spiky", 8, 16, 16, 4096, 64, True,
                spike_frac=0.01, spike_mult=8.0, seed=1003),
    4: Workload("gqa_causal", 1, 32, 8, 8192, 256, True, seed=1004),
    5: Workload("long_context_mqa_causal", 1, 32, 1, 131072, 128, True,
                sigma=0.5, sample_rows=256, seed=1005),
}


def _draw(rng, B, H, N, d, sigma, spike_frac, spike_mult) -> np.ndarray:
    out = np.empty((B, H, N, d), dtype=np.float16)
    spikes = None
    need_spikes = spike_frac > 0.0
    full = np.empty((B, H, N, d), dtype=np.float32) if need_spikes else None
    for b in range(B):
        for h in range(H):
            x = rng.standard_normal((N, d), dtype=np.float32)
            if sigma != 1.0:
                x *= np.float32(sigma)
            if need_spikes:
                full[b, h] = x
            else:
                out[b, h] = x.astype(np.float16)
    if need_spikes:
        count = int(round(spike_frac * B * H * N))
        spikes = rng.choice(B * H * N, size=count, replace=False)
        flat = full.reshape(B * H * N, d)
        flat[spikes] *= np.float32(spike_mult)
        out[...] = full.astype(np.float16)
    return out


def make_qkv(B, Hq, Hkv, N, d, seed, sigma=1.0, spike_frac=0.0, spike_mult=1.0):
    """Q [B,Hq,N,d], K/V [B,Hkv,N,d] as fp16 numpy arrays, per the recipe."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, B, Hq, N, d, sigma, spike_frac, spike_mult)
    k = _draw(rng, B, Hkv, N, d, sigma, spike_frac, spike_mult)
    v = _draw(rng, B, Hkv, N, d, sigma, 0.0, 1.0)
    return q, k, v


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bfloat16 (ties to even), returned as
    fp32 (every bf16 value is exactly an fp32 value).  NaN/Inf are not drawn."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bits = (bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return bits.view(np.float32)


def make_qkv_bf16(B, Hq, Hkv, N, d, seed, sigma=1.0, spike_frac=0.0, spike_mult=1.0):
    """Q, K, V as make_qkv draws them (same generator calls), rounded to
    bfloat16 instead of fp16; fp32 arrays holding bf16 values."""
    rng = np.random.default_rng(seed)
    out = []
    for H, spiky in ((Hq, True), (Hkv, True), (Hkv, False)):
        full = np.empty((B, H, N, d), dtype=np.float32)
        for b in range(B):
            for h in range(H):
                x = rng.standard_normal((N, d), dtype=np.float32)
                if sigma != 1.0:
                    x *= np.float32(sigma)
                full[b, h] = x
        if spiky and spike_frac > 0.0:
            count = int(round(spike_frac * B * H * N))
            rows = rng.choice(B * H * N, size=count, replace=False)
            full.reshape(B * H * N, d)[rows] *= np.float32(spike_mult)
        out.append(round_to_bf16(full))
    return tuple(out)


def make_inputs(w: Workload, seed: int | None = None):
    """Inputs of a named workload (its own seed unless one is given)."""
    s = w.seed if seed is None else seed
    return make_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, s, w.sigma, w.spike_frac, w.spike_mult)


def sample_rows(w: Workload, count: int | None = None, seed: int | None = None) -> np.ndarray:
    """Query rows the oracle checks per head: [B, Hq, R] int64, sorted.

    Rows 0 and N-1 are always included (both ends of the causal range).
    """
    R = count if count is not None else w.sample_rows
    s = w.seed if seed is None else seed
    N = w.N
    R = min(R, N)
    out = np.empty((w.B, w.Hq, R), dtype=np.int64)
    for b in range(w.B):
        for hq in range(w.Hq):
            if R == N:
                out[b, hq] = np.arange(N)
                continue
            rng = np.random.default_rng(s + 10**6 + b * w.Hq + hq)
            inner = rng.choice(np.arange(1, N - 1), size=R - 2, replace=False)
            out[b, hq] = np.sort(np.concatenate([[0, N - 1], inner]))
    return out


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Nq new queries (the last Nq positions) against a cache of Nk keys/values."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool = True
    sigma: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic bytes: K and V read once, Q read once, O (fp16) and LSE (fp32) written once."""
        kv = 2 * self.B * self.Hkv * self.Nk * self.d * 2
        q_o = 2 * self.B * self.Hq * self.Nq * self.d * 2
        return kv + q_o + self.B * self.Hq * self.Nq * 4

    def describe(self) -> str:
        mask = "causal" if self.causal else "non-causal"
        return f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} Nq={self.Nq} Nk={self.Nk} d={self.d} {mask}"


DECODE_WORKLOADS = {
    1: DecodeWorkload("gqa_decode_batch64", 64, 32, 8, 1, 8192, 128, seed=2001),
    2: DecodeWorkload("long_context_mqa_decode", 1, 32, 1, 1, 131072, 128, sigma=0.5, seed=2002),
    3: DecodeWorkload("gqa_d256_decode", 1, 32, 8, 1, 8192, 256, seed=2003),
    4: DecodeWorkload("multi_query_decode", 4, 32, 8, 16, 8192, 128, seed=2004),
}


def make_decode_qkv(B, Hq, Hkv, Nq, Nk, d, seed, sigma=1.0):
    """Q [B,Hq,Nq,d], K/V [B,Hkv,Nk,d] as fp16 numpy arrays, per the recipe."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, B, Hq, Nq, d, sigma, 0.0, 1.0)
    k = _draw(rng, B, Hkv, Nk, d, sigma, 0.0, 1.0)
    v = _draw(rng, B, Hkv, Nk, d, sigma, 0.0, 1.0)
    return q, k, v


def make_decode_inputs(w: DecodeWorkload, seed: int | None = None):
    s = w.seed if seed is None else seed
    return make_decode_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, s, w.sigma)
