"""Plain fp64 attention forward on the CPU (test infrastructure only).

This is the oracle the GPU path is checked against.  It is written to be read
against the pages, not to be fast: every step below is one line of the
definition, with no blocking, fusion or reordering beyond what the pages
state.  Only the test suite, ``__graft_entry__.smoke`` and the ``cpu_baseline``
leg of ``bench.py`` may use it; the product path never does.

Pages cited:
  [CANN-FA]  www.mooersco.com/news/1200175, "FlashAttention operator of the CANN
             ops-transformer repository: attention acceleration on the Ascend NPU"
  [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html (the "dictionary,
             page by page" FlashAttention tutorial)
  [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html (why Transformer
             inference is slow; FlashAttention on Ascend / CANN)

What is computed ([CANN-FA] section "Where is the bottleneck of standard
attention"; [FA-Infer] section 2, "Where the compute bottleneck of attention
lies"): S = Q K^T, P = softmax(S) by rows, O = P V.  The pages scale the
logits by 1/sqrt(head_dim) ([FA-Dict] section "Fused kernel", the Scale call;
[FA-Dict] section "Calling", attn_scale=1/sqrt(128)) and use a causal mask
through SDPA's is_causal flag ([CANN-FA] section "Calling FlashAttention from
PyTorch").  The softmax is taken in two passes: first the row maximum, then
the exponentials, their sum and the division ([CANN-FA], the paragraph after
"Tiling on the Ascend NPU" that contrasts ordinary two-pass softmax with the
online form).

Readings taken where the pages are silent (each also listed in the design
notes of the repository):
  * The scale is an fp32 number at the library boundary; the oracle uses that
    very fp32 value, widened exactly to fp64.
  * Causal means key j is visible to query i iff j <= i (queries and keys have
    the same length, so top-left and bottom-right alignment coincide).  A
    masked key has weight exactly 0.
  * GQA/MQA ([FA-Infer] section 6): query heads are split into Hkv contiguous
    groups of G = Hq/Hkv; query head h reads key/value head h // G.
  * LSE is the natural log of the sum of exp over the visible scaled logits.
  * Inputs are widened exactly to fp64; all arithmetic is fp64.

The online-softmax recurrence ([CANN-FA] section "Concrete flow", step 3, and
the comments of its Ascend C kernel; [FA-Dict] section "Online softmax") is
also written out here, as scalar Python loops generic over the number type,
so that tests can prove it equal to the two-pass form in exact-enough
arithmetic.  It is never used to produce an expected value for the GPU.
"""

from __future__ import annotations

import math

import numpy as np


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head ``hq``.

    [FA-Infer] section 6 says the operator supports GQA and MQA; the pages do
    not fix the grouping.  Reading: Hkv contiguous groups of G = Hq/Hkv query
    heads (MHA: G = 1, MQA: Hkv = 1).
    """
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    group = Hq // Hkv
    return hq // group


def _fp32_scale(scale: float) -> float:
    """The boundary takes the scale as an fp32 number; widen that exactly."""
    return float(np.float32(scale))


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float,
                    causal: bool = False) -> np.ndarray:
    """P = softmax(scale * Q K^T) for ONE head, as an N_q x N matrix in fp64.

    q: [Nq, d], k: [N, d].  Query i sees key j iff (not causal) or j <= i.
    Two passes: row max, then exponentials, their sum and the division
    ([CANN-FA], paragraph on ordinary two-pass softmax).
    """
    q64 = np.asarray(q).astype(np.float64)
    k64 = np.asarray(k).astype(np.float64)
    sigma = _fp32_scale(scale)
    S = sigma * (q64 @ k64.T)
    if causal:
        i = np.arange(q64.shape[0])[:, None]
        j = np.arange(k64.shape[0])[None, :]
        S = np.where(j <= i, S, -np.inf)
    m = S.max(axis=1)                  # pass 1: row maximum
    E = np.exp(S - m[:, None])         # pass 2: exponentials (masked -> 0)
    l = E.sum(axis=1)                  #         their sum
    return E / l[:, None]              #         normalisation


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  causal: bool = False, rows=None, max_chunk_elems: int = 1 << 24):
    """Two-pass fp64 attention over a batch of heads.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float dtype, widened exactly).
    rows: None for every query row; a 1-D integer array for the same query rows
    in every (b, hq); or an integer array [B, Hq, R] of rows per head.
    Returns (O [B, Hq, R, d] fp64, LSE [B, Hq, R] fp64).

    For each (b, hq) and each query row i, with kvh = kv_head_of(hq):
      s_ij   = scale * q_i . k_j                  (for every key j)
      m_i    = max over visible j of s_ij         (pass 1)
      e_ij   = exp(s_ij - m_i), 0 when masked     (pass 2)
      l_i    = sum_j e_ij
      O_i    = sum_j (e_ij / l_i) v_j
      LSE_i  = m_i + ln l_i
    Rows are processed in chunks only to bound memory; each row's arithmetic
    is the same whatever the chunk.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape[:3] != (B, Hkv, N):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    dv = v.shape[3]
    sigma = _fp32_scale(scale)

    if rows is None:
        rows_of = lambda b, h: np.arange(N)  # noqa: E731
        R = N
    else:
        rows = np.asarray(rows, dtype=np.int64)
        if rows.ndim == 1:
            rows_of = lambda b, h: rows  # noqa: E731
            R = rows.shape[0]
        else:
            if rows.shape[:2] != (B, Hq):
                raise ValueError("rows must be [R] or [B, Hq, R]")
            rows_of = lambda b, h: rows[b, h]  # noqa: E731
            R = rows.shape[2]

    O = np.empty((B, Hq, R, dv), dtype=np.float64)
    LSE = np.empty((B, Hq, R), dtype=np.float64)
    chunk = max(1, min(R, max_chunk_elems // max(N, 1)))
    keys = np.arange(N)[None, :]
    for b in range(B):
        for hq in range(Hq):
            kvh = kv_head_of(hq, Hq, Hkv)
            K = k[b, kvh].astype(np.float64)
            V = v[b, kvh].astype(np.float64)
            rr = rows_of(b, hq)
            for c0 in range(0, R, chunk):
                ri = rr[c0:c0 + chunk]
                Qc = q[b, hq, ri].astype(np.float64)
                S = sigma * (Qc @ K.T)
                if causal:
                    S = np.where(keys <= ri[:, None], S, -np.inf)
                m = S.max(axis=1)
                E = np.exp(S - m[:, None])
                l = E.sum(axis=1)
                P = E / l[:, None]
                O[b, hq, c0:c0 + len(ri)] = P @ V
                LSE[b, hq, c0:c0 + len(ri)] = m + np.log(l)
    return O, LSE


def attention_decode_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                         causal: bool = True):
    """Two-pass fp64 attention for a decode (KV-cache) step.

    q: [B, Hq, Nq, d] are the last Nq positions of a sequence whose keys and
    values k, v: [B, Hkv, Nk, d] (Nq <= Nk) cover all Nk positions.  Same
    definition as ``attention_ref`` ([CANN-FA] section "Where is the
    bottleneck of standard attention"; [FA-Infer] section 2); the only new
    reading is where the queries sit: query i is position Nk - Nq + i, so
    with ``causal`` it sees keys j <= Nk - Nq + i (with Nq == Nk this is the
    causal mask of ``attention_ref``).  GQA/MQA grouping as ``kv_head_of``
    ([FA-Infer] section 6, which ties GQA/MQA to the KV cache of inference).
    Returns (O [B, Hq, Nq, d] fp64, LSE [B, Hq, Nq] fp64).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape[:3] != (B, Hkv, Nk) or Nq > Nk:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    sigma = _fp32_scale(scale)
    pos = (Nk - Nq) + np.arange(Nq)          # position of each query in the sequence
    keys = np.arange(Nk)
    O = np.empty((B, Hq, Nq, v.shape[3]), dtype=np.float64)
    LSE = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            kvh = kv_head_of(hq, Hq, Hkv)
            K = k[b, kvh].astype(np.float64)
            V = v[b, kvh].astype(np.float64)
            S = sigma * (q[b, hq].astype(np.float64) @ K.T)    # [Nq, Nk]
            if causal:
                S = np.where(keys[None, :] <= pos[:, None], S, -np.inf)
            m = S.max(axis=1)                                  # pass 1
            E = np.exp(S - m[:, None])                         # pass 2
            l = E.sum(axis=1)
            O[b, hq] = (E / l[:, None]) @ V
            LSE[b, hq] = m + np.log(l)
    return O, LSE


def online_attention(q, k, v, scale, causal=False, blocks=None,
                     normalise_each_step=True, num=float, exp=math.exp,
                     log=math.log):
    """The online-softmax recurrence for ONE head, as scalar loops.

    Follows [CANN-FA] section "Concrete flow": for each query row, visit the
    key blocks in the given order and keep a running maximum m and a running
    exponential sum l.  With the stripped operators of that section restored
    (the only dimensionally consistent reading):
        m_new   = max(m_old, max_j S_block)
        l_new   = l_old * exp(m_old - m_new) + sum_j exp(S_block - m_new)
    normalise_each_step=True is the section's per-block form:
        P_block = exp(S_block - m_new) / l_new
        O       = O * (l_old * exp(m_old - m_new) / l_new) + P_block V_block
    normalise_each_step=False is the "normalise once at the end" form the same
    page describes (and [FA-Dict] section "Online softmax"):
        A       = A * exp(m_old - m_new) + exp(S_block - m_new) V_block
        O       = A / l        after the last block.
    LSE = m + ln l.

    q: Nq x d, k: N x d, v: N x dv, as nested sequences or arrays; each element
    is converted with ``num``.  ``blocks`` is a list of lists of key indices
    (default: contiguous blocks of two keys in ascending order); any partition
    of the keys, in any order, is allowed.  A block with no key visible to the
    row contributes nothing: with every logit masked to -inf, max leaves m
    unchanged and every exp is 0 (when m_old is still -inf this is the guard
    that replaces exp(-inf - (-inf))).

    ``num``, ``exp`` and ``log`` select the arithmetic (Python floats by
    default; mpmath's mpf/exp/log for high precision).
    """
    Q = [[num(float(x)) for x in row] for row in np.asarray(q, dtype=np.float64)]
    Kt = [[num(float(x)) for x in row] for row in np.asarray(k, dtype=np.float64)]
    Vt = [[num(float(x)) for x in row] for row in np.asarray(v, dtype=np.float64)]
    sigma = num(_fp32_scale(scale))
    N = len(Kt)
    dv = len(Vt[0]) if N else 0
    if blocks is None:
        blocks = [list(range(j, min(j + 2, N))) for j in range(0, N, 2)]
    covered = sorted(j for blk in blocks for j in blk)
    if covered != list(range(N)):
        raise ValueError("blocks must partition the keys 0..N-1")

    O_out, L_out = [], []
    neg_inf = num(float("-inf"))
    zero = num(0)
    for i, qi in enumerate(Q):
        m = neg_inf
        l = zero
        o = [zero] * dv
        for blk in blocks:
            js = [j for j in blk if (not causal) or j <= i]
            if not js:
                continue
            s = [sigma * sum(a * b for a, b in zip(qi, Kt[j])) for j in js]
            m_new = max([m] + s)
            corr = exp(m - m_new)
            e = [exp(x - m_new) for x in s]
            l_new = l * corr + sum(e)
            if normalise_each_step:
                p = [et / l_new for et in e]
                keep = l * corr / l_new
                o = [o[c] * keep + sum(p[t] * Vt[j][c] for t, j in enumerate(js))
                     for c in range(dv)]
            else:
                o = [o[c] * corr + sum(e[t] * Vt[j][c] for t, j in enumerate(js))
                     for c in range(dv)]
            m, l = m_new, l_new
        if not normalise_each_step:
            o = [x / l for x in o]
        O_out.append(o)
        L_out.append(m + log(l))
    return O_out, L_out
