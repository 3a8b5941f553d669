"""Plain fp64 attention backward on the CPU (test infrastructure only).

The gradients of the attention forward with respect to its inputs, as the
oracle the GPU backward is checked against.  Only the test suite and the
``cpu_baseline`` leg of ``bench.py`` may use it; the product path never does.

Pages cited:
  [CANN-FA]  www.mooersco.com/news/1200175, "FlashAttention operator of the CANN
             ops-transformer repository: attention acceleration on the Ascend NPU"
  [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html
  [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html

The pages name training as a use of the operator ([CANN-FA], opening
paragraph: the self-attention layer is the bottleneck of large-model
inference and training) and note that backpropagation must also keep
gradients ([FA-Dict] section "Standard attention"), but they do not write the
backward pass out.  It is fixed by the forward definition alone
([CANN-FA] section "Where is the bottleneck of standard attention":
S = Q K^T scaled, P = softmax(S) by rows, O = P V) and the chain rule: for an
upstream gradient dO of O, with sigma the fp32 scale widened exactly,

    dV   = P^T dO                       (O is linear in V)
    dP   = dO V^T                       (O is linear in P)
    dS_ij = P_ij (dP_ij - sum_t P_it dP_it)
                                        (Jacobian of a row softmax; masked
                                         entries have P = 0, so dS = 0)
    dQ   = sigma dS K,   dK = sigma dS^T Q
                                        (S = sigma Q K^T)

Readings: the same masking, GQA grouping and scale conventions as
``oracle.attention`` (a key/value head's gradient is the sum over the query
heads that read it); the loss is whatever produced dO, so only dO enters;
LSE is an output of the forward, not an input here, so its gradient is not
part of this definition.
"""

from __future__ import annotations

import numpy as np

from .attention import _fp32_scale, attention_probs, kv_head_of


def attention_bwd_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                      causal: bool = False):
    """Exact (fp64) gradients (dQ, dK, dV) of O = softmax(scale Q K^T [+mask]) V.

    q, do: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float dtype, widened
    exactly).  Returns fp64 arrays shaped like q, k, v.  P is the two-pass
    softmax of ``attention_probs``; every other line is one line of the chain
    rule above.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape[:3] != (B, Hkv, N) or do.shape != q.shape[:3] + (v.shape[3],):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape} do{do.shape}")
    sigma = _fp32_scale(scale)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            kvh = kv_head_of(hq, Hq, Hkv)
            Q = q[b, hq].astype(np.float64)
            K = k[b, kvh].astype(np.float64)
            V = v[b, kvh].astype(np.float64)
            dO = do[b, hq].astype(np.float64)
            P = attention_probs(Q, K, scale, causal=causal)          # [N, N]
            dv[b, kvh] += P.T @ dO
            dP = dO @ V.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, hq] = sigma * (dS @ K)
            dk[b, kvh] += sigma * (dS.T @ Q)
    return dq, dk, dv


def attention_bwd_delta(o: np.ndarray, do: np.ndarray) -> np.ndarray:
    """Delta_i = sum_c dO_ic O_ic per query row, [B, H, N] fp64.

    With the exact O this equals sum_t P_it dP_it of the chain rule (since
    O_i = sum_t P_it V_t); the GPU computes it from the fp16 O the forward
    stored.  Used only by tests that check that step on its own.
    """
    return (np.asarray(o).astype(np.float64) * np.asarray(do).astype(np.float64)).sum(axis=-1)
