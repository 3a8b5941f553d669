"""Pins of the backward oracle (oracle/backward.py) against what the forward
definition and the mathematics fix, independently of the chain-rule lines
being checked.

Every pin takes the module under test (``impl``) so that the mutation test
can run the same pins against copies of the oracle with a planted mistake.
The forward oracle (oracle.attention, pinned on its own) provides O for the
finite differences; torch's autograd provides a second, library-made
gradient.
"""

from __future__ import annotations

import numpy as np

from oracle.attention import attention_probs, attention_ref


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert (err <= lim).all(), f"{what}: max err {err.max():.3e} (limit {lim.max():.3e})"


def _loss(q, k, v, do, scale, causal):
    O, _ = attention_ref(q, k, v, scale, causal=causal)
    return float((O * do).sum())


def pin_bwd_finite_differences(impl):
    """Central differences of L = sum(dO * O), with O from the forward
    oracle, match the analytic gradients for every input element."""
    rng = _rng(31)
    for Hq, Hkv, N, d, causal in ((2, 1, 5, 3, False), (2, 1, 5, 3, True), (1, 1, 1, 2, False),
                                  (4, 2, 4, 2, True)):
        q, k, v = _rand(rng, 1, Hq, N, d), _rand(rng, 1, Hkv, N, d), _rand(rng, 1, Hkv, N, d)
        do = _rand(rng, 1, Hq, N, d)
        scale = 0.7
        dq, dk, dv = impl.attention_bwd_ref(q, k, v, do, scale, causal=causal)
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy()
                xp[idx] += h
                lp = _loss(*(xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))), do, scale, causal)
                xp[idx] -= 2 * h
                lm = _loss(*(xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))), do, scale, causal)
                num[idx] = (lp - lm) / (2 * h)
            _close(g, num, 1e-6, 1e-7, f"d{name} vs finite differences (Hq={Hq} Hkv={Hkv} N={N} causal={causal})")


def pin_bwd_torch_autograd(impl):
    """torch's autograd in fp64 on the CPU (explicit softmax(scale QK^T) V,
    K/V heads repeated for GQA) gives the same gradients."""
    import torch
    rng = _rng(32)
    for Hq, Hkv, N, d, causal in ((4, 2, 9, 6, True), (3, 3, 7, 5, False), (4, 1, 11, 4, True)):
        q, k, v = _rand(rng, 2, Hq, N, d), _rand(rng, 2, Hkv, N, d), _rand(rng, 2, Hkv, N, d)
        do = _rand(rng, 2, Hq, N, d)
        scale = float(np.float32(0.37))
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        G = Hq // Hkv
        kr = tk.repeat_interleave(G, dim=1)
        vr = tv.repeat_interleave(G, dim=1)
        s = scale * torch.matmul(tq, kr.transpose(-1, -2))
        if causal:
            mask = torch.ones(N, N, dtype=torch.bool).tril()
            s = s.masked_fill(~mask, float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), vr)
        o.backward(torch.tensor(do))
        dq, dk, dv = impl.attention_bwd_ref(q, k, v, do, scale, causal=causal)
        _close(dq, tq.grad.numpy(), 1e-10, 1e-12, "dq vs torch autograd")
        _close(dk, tk.grad.numpy(), 1e-10, 1e-12, "dk vs torch autograd")
        _close(dv, tv.grad.numpy(), 1e-10, 1e-12, "dv vs torch autograd")


def pin_bwd_key_shift_invariance(impl):
    """Adding one vector to every key adds q_i.u to every visible logit of
    row i, which the softmax ignores: the gradient along that direction,
    sum_j dK_j, is 0 for each key/value head (causal or not)."""
    rng = _rng(33)
    for causal in (False, True):
        q, k, v = _rand(rng, 2, 4, 8, 5), _rand(rng, 2, 2, 8, 5), _rand(rng, 2, 2, 8, 5)
        do = _rand(rng, 2, 4, 8, 5)
        _, dk, _ = impl.attention_bwd_ref(q, k, v, do, 0.9, causal=causal)
        _close(dk.sum(axis=2), np.zeros((2, 2, 5)), 0, 1e-12, f"sum_j dK_j causal={causal}")


def pin_bwd_dv_sums_to_do(impl):
    """Rows of P sum to 1, so sum_j dV_j = sum over the head's query heads
    and rows of dO."""
    rng = _rng(34)
    for causal in (False, True):
        q, k, v = _rand(rng, 1, 6, 7, 3), _rand(rng, 1, 2, 7, 3), _rand(rng, 1, 2, 7, 4)
        do = _rand(rng, 1, 6, 7, 4)
        _, _, dv = impl.attention_bwd_ref(q, k, v, do, 1.3, causal=causal)
        want = do.reshape(1, 2, 3, 7, 4).sum(axis=(2, 3))
        _close(dv.sum(axis=2), want, 1e-12, 1e-12, f"sum_j dV_j causal={causal}")


def pin_bwd_scale_zero(impl):
    """scale 0: S is constant, so dQ = dK = 0 exactly and dV_j is the sum of
    dO_i / (number of keys row i sees) over the rows that see key j."""
    rng = _rng(35)
    N = 6
    q, k, v = _rand(rng, 1, 2, N, 3), _rand(rng, 1, 1, N, 3), _rand(rng, 1, 1, N, 3)
    do = _rand(rng, 1, 2, N, 3)
    for causal in (False, True):
        dq, dk, dv = impl.attention_bwd_ref(q, k, v, do, 0.0, causal=causal)
        assert not dq.any() and not dk.any(), "scale 0: dQ and dK must be exactly 0"
        want = np.zeros((N, 3))
        for h in range(2):
            for i in range(N):
                seen = range(i + 1) if causal else range(N)
                for j in seen:
                    want[j] += do[0, h, i] / len(seen)
        _close(dv[0, 0], want, 1e-13, 1e-14, f"scale 0 dV causal={causal}")


def pin_bwd_single_key(impl):
    """One key: P = 1 whatever the logits, so dS = 0 (dQ = dK = 0) and
    dV = the sum of dO over the query heads."""
    rng = _rng(36)
    q, k, v = _rand(rng, 1, 3, 1, 4), _rand(rng, 1, 1, 1, 4), _rand(rng, 1, 1, 1, 4)
    do = _rand(rng, 1, 3, 1, 4)
    dq, dk, dv = impl.attention_bwd_ref(q, k, v, do, 0.8, causal=True)
    _close(dq, np.zeros_like(dq), 0, 1e-15, "N=1 dQ")
    _close(dk, np.zeros_like(dk), 0, 1e-15, "N=1 dK")
    _close(dv[0, 0, 0], do[0, :, 0].sum(axis=0), 1e-15, 1e-15, "N=1 dV")


def pin_bwd_gqa_is_summed_mha(impl):
    """GQA equals MHA on K/V heads repeated G times, with each key/value
    head's gradient the sum over its G copies."""
    rng = _rng(37)
    G, Hkv, N, d = 3, 2, 6, 4
    q, k, v = _rand(rng, 2, G * Hkv, N, d), _rand(rng, 2, Hkv, N, d), _rand(rng, 2, Hkv, N, d)
    do = _rand(rng, 2, G * Hkv, N, d)
    for causal in (False, True):
        dq, dk, dv = impl.attention_bwd_ref(q, k, v, do, 0.5, causal=causal)
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        dq2, dk2, dv2 = impl.attention_bwd_ref(q, kr, vr, do, 0.5, causal=causal)
        _close(dq, dq2, 1e-13, 1e-14, "GQA dQ")
        _close(dk, dk2.reshape(2, Hkv, G, N, d).sum(axis=2), 1e-13, 1e-14, "GQA dK")
        _close(dv, dv2.reshape(2, Hkv, G, N, d).sum(axis=2), 1e-13, 1e-14, "GQA dV")


def pin_bwd_delta_identity(impl):
    """sum_t P_it dP_it = dO_i . O_i (O_i = sum_t P_it V_t): the quantity the
    GPU takes from the stored O."""
    rng = _rng(38)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4)
    do = _rand(rng, 1, 2, 9, 4)
    for causal in (False, True):
        O, _ = attention_ref(q, k, v, 0.6, causal=causal)
        got = impl.attention_bwd_delta(O, do)
        for h in range(2):
            P = attention_probs(q[0, h], k[0, h], 0.6, causal=causal)
            want = (P * (do[0, h] @ v[0, h].T)).sum(axis=1)
            _close(got[0, h], want, 1e-12, 1e-13, f"delta identity causal={causal}")


BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_torch_autograd,
    pin_bwd_key_shift_invariance,
    pin_bwd_dv_sums_to_do,
    pin_bwd_scale_zero,
    pin_bwd_single_key,
    pin_bwd_gqa_is_summed_mha,
    pin_bwd_delta_identity,
]
