"""Textbook attention as scalar loops over mpmath numbers (test infrastructure only).

For tiny inputs only.  This is the softmax definition itself,
    softmax(s)_j = exp(s_j) / sum_t exp(s_t),
with no subtraction of a running or row maximum, evaluated at ``dps`` decimal
digits, so that it shares neither the stabilisation trick nor the numpy/BLAS
arithmetic of ``oracle.attention``.  It pins that module and the online
recurrence in the tests.

Pages cited: [CANN-FA] www.mooersco.com/news/1200175, section "Where is the
bottleneck of standard attention" (S = Q K^T, P = softmax(S) by rows, O = P V);
[FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html, section 2 (the
same three steps); [FA-Infer] section 6 for GQA/MQA (grouping reading: query
head h reads key/value head h // (Hq/Hkv)).
"""

from __future__ import annotations

import mpmath
import numpy as np


def attention_brute(q, k, v, scale, causal=False, dps=50):
    """O and LSE for q [B,Hq,Nq,d], k/v [B,Hkv,N,d] as nested lists of mpf.

    Every input element is converted exactly (binary floats are exact in
    mpmath).  The scale is taken as the fp32 number the library boundary
    receives.  The Nq queries are the last Nq of the N positions (Nq = N for
    ordinary attention): query i sees key j iff (not causal) or
    j <= N - Nq + i.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    shift = N - Nq
    G = Hq // Hkv
    with mpmath.workdps(dps):
        sigma = mpmath.mpf(float(np.float32(scale)))
        O = []
        LSE = []
        for b in range(B):
            Ob, Lb = [], []
            for h in range(Hq):
                g = h // G
                Oh, Lh = [], []
                for i in range(Nq):
                    weights = []
                    for j in range(N):
                        if causal and j > shift + i:
                            continue
                        dot = mpmath.mpf(0)
                        for c in range(d):
                            dot += mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, g, j, c])
                        weights.append((j, mpmath.exp(sigma * dot)))
                    total = mpmath.fsum(w for _, w in weights)
                    row = []
                    for c in range(v.shape[3]):
                        row.append(mpmath.fsum(w * mpmath.mpf(v[b, g, j, c])
                                               for j, w in weights) / total)
                    Oh.append(row)
                    Lh.append(mpmath.log(total))
                Ob.append(Oh)
                Lb.append(Lh)
            O.append(Ob)
            LSE.append(Lb)
    return O, LSE


def to_float_array(nested) -> np.ndarray:
    """Round a nested list of mpf to an fp64 numpy array."""
    return np.array(nested, dtype=object).astype(np.float64)
