"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an oracle implementation (the ``oracle.attention``
module, or a deliberately broken copy of it in the mutation tests) and raises
AssertionError when the implementation disagrees with something other than
itself: a closed form, an invariant of the softmax definition, a brute-force
evaluation of the textbook definition in high precision, or torch's CPU
scaled_dot_product_attention (secondary).

Pages cited:
  [CANN-FA]  www.mooersco.com/news/1200175 (FlashAttention operator of CANN
             ops-transformer on the Ascend NPU)
  [FA-Dict]  hwcomputing.csdn.net/6a0dbd08662f9a54cb75eb74.html
  [FA-Infer] gitcode.csdn.net/6a0c62d2662f9a54cb75b31f.html
"""

from __future__ import annotations

import itertools
import json
import math
import os

import mpmath
import numpy as np

from oracle.brute import attention_brute, to_float_array

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    bad = err > lim
    assert not bad.any(), f"{what}: max err {err.max():.3e} (first bad at {np.argwhere(bad)[0]})"


# ---------------------------------------------------------------------------
# Closed forms written down by hand (tests/golden/closed_forms.json)
# ---------------------------------------------------------------------------

def pin_golden_closed_forms(impl):
    """Hand-derived outputs of tiny problems; see the fixture for derivations."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(c[t], dtype=np.float64) for t in ("q", "k", "v"))
        for causal, key in ((False, "noncausal"), (True, "causal")):
            O, L = impl.attention_ref(q, k, v, c["scale"], causal=causal)
            _close(O, c[key]["O"], 1e-13, 1e-15, f"{c['name']} {key} O")
            _close(L, c[key]["LSE"], 1e-13, 1e-15, f"{c['name']} {key} LSE")


# ---------------------------------------------------------------------------
# Brute force: the textbook definition at 40 digits, no max subtraction
# ---------------------------------------------------------------------------

def pin_brute_force_small(impl):
    """numpy two-pass oracle == mpmath textbook softmax for N <= 8."""
    rng = _rng(7)
    for N, d, (Hq, Hkv), causal in itertools.product(
            (1, 2, 3, 5, 8), (1, 2, 4), ((1, 1), (2, 1), (4, 2)), (False, True)):
        q = _rand(rng, 1, Hq, N, d)
        k = _rand(rng, 1, Hkv, N, d)
        v = _rand(rng, 1, Hkv, N, d)
        scale = 0.7
        O, L = impl.attention_ref(q, k, v, scale, causal=causal)
        Ob, Lb = attention_brute(q, k, v, scale, causal=causal, dps=40)
        _close(O, to_float_array(Ob), 1e-12, 1e-13, f"brute O N={N} d={d} H={Hq}/{Hkv} c={causal}")
        _close(L, to_float_array(Lb), 1e-12, 1e-13, f"brute LSE N={N} d={d} H={Hq}/{Hkv} c={causal}")


def pin_probs_brute_force(impl):
    """attention_probs == exp(s_ij) / sum_t exp(s_it) from mpmath, masked entries 0."""
    rng = _rng(8)
    for N, causal in itertools.product((1, 3, 6), (False, True)):
        q = _rand(rng, N, 3)
        k = _rand(rng, N, 3)
        P = impl.attention_probs(q, k, 0.9, causal=causal)
        sigma = mpmath.mpf(float(np.float32(0.9)))
        with mpmath.workdps(40):
            for i in range(N):
                vis = [j for j in range(N) if not causal or j <= i]
                w = {j: mpmath.exp(sigma * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b)
                                                       for a, b in zip(q[i], k[j])))
                     for j in vis}
                tot = mpmath.fsum(w.values())
                for j in range(N):
                    want = float(w[j] / tot) if j in w else 0.0
                    got = P[i, j]
                    if j not in w:
                        assert got == 0.0, f"masked P[{i},{j}] = {got}"
                    else:
                        assert abs(got - want) <= 1e-14 + 1e-13 * abs(want), \
                            f"P[{i},{j}] {got} vs {want}"


# ---------------------------------------------------------------------------
# The online recurrence of the pages equals the two-pass form
# ---------------------------------------------------------------------------

def _mp_online(impl, q, k, v, scale, causal, blocks, each_step):
    return impl.online_attention(q, k, v, scale, causal=causal, blocks=blocks,
                                 normalise_each_step=each_step, num=mpmath.mpf,
                                 exp=mpmath.exp, log=mpmath.log)


def pin_online_equals_two_pass_exact(impl):
    """Both online forms == textbook definition to < 1e-50 at 60 digits.

    [FA-Dict] section "Online softmax" and [FA-Infer] section 3 state that the
    online result is exactly the standard softmax result; read as exact
    arithmetic, checked here at 60 significant digits.
    """
    rng = _rng(9)
    with mpmath.workdps(60):
        for N, d, causal in ((1, 2, False), (4, 3, False), (5, 2, True), (6, 3, True)):
            q = _rand(rng, N, d)
            k = _rand(rng, N, d)
            v = _rand(rng, N, 2)
            Ob, Lb = attention_brute(q[None, None], k[None, None], v[None, None],
                                     0.8, causal=causal, dps=60)
            for blocks in ([list(range(N))],
                           [[j] for j in range(N)],
                           [list(range(j, min(j + 2, N))) for j in range(0, N, 2)],
                           [[j] for j in reversed(range(N))]):
                for each_step in (True, False):
                    O, L = _mp_online(impl, q, k, v, 0.8, causal, blocks, each_step)
                    for i in range(N):
                        assert abs(L[i] - Lb[0][0][i]) < mpmath.mpf(10) ** -50, "online LSE"
                        for c in range(2):
                            assert abs(O[i][c] - Ob[0][0][i][c]) < mpmath.mpf(10) ** -50, \
                                f"online O N={N} causal={causal} blocks={blocks} each={each_step}"


def _compositions(N):
    """Every split of 0..N-1 into contiguous blocks (2^(N-1) of them)."""
    for cuts in itertools.product((False, True), repeat=max(N - 1, 0)):
        blocks, cur = [], [0]
        for j in range(1, N):
            if cuts[j - 1]:
                blocks.append(cur)
                cur = []
            cur.append(j)
        blocks.append(cur)
        yield blocks


def pin_online_block_invariance(impl):
    """fp64 online forms agree with the two-pass oracle for EVERY contiguous
    block split (N <= 6) and every visiting order of single-key blocks (N <= 5),
    and on a random sample of orders for N = 8."""
    rng = _rng(10)
    for N, causal in ((3, False), (5, True), (6, False), (6, True)):
        q, k, v = _rand(rng, N, 2), _rand(rng, N, 2), _rand(rng, N, 3)
        O_ref, L_ref = impl.attention_ref(q[None, None], k[None, None], v[None, None],
                                          1.1, causal=causal)
        for blocks in _compositions(N):
            for each in (True, False):
                O, L = impl.online_attention(q, k, v, 1.1, causal=causal, blocks=blocks,
                                             normalise_each_step=each)
                _close(O, O_ref[0, 0], 1e-13, 1e-14, f"split {blocks}")
                _close(L, L_ref[0, 0], 1e-13, 1e-14, f"split {blocks} LSE")
    for N, causal in ((4, True), (5, False)):
        q, k, v = _rand(rng, N, 2), _rand(rng, N, 2), _rand(rng, N, 2)
        O_ref, L_ref = impl.attention_ref(q[None, None], k[None, None], v[None, None],
                                          0.6, causal=causal)
        for order in itertools.permutations(range(N)):
            O, L = impl.online_attention(q, k, v, 0.6, causal=causal,
                                         blocks=[[j] for j in order],
                                         normalise_each_step=bool(order[0] % 2))
            _close(O, O_ref[0, 0], 1e-13, 1e-14, f"order {order}")
            _close(L, L_ref[0, 0], 1e-13, 1e-14, f"order {order} LSE")
    N = 8
    q, k, v = _rand(rng, N, 2), _rand(rng, N, 2), _rand(rng, N, 2)
    O_ref, L_ref = impl.attention_ref(q[None, None], k[None, None], v[None, None], 0.6,
                                      causal=True)
    for _ in range(60):
        order = rng.permutation(N)
        O, L = impl.online_attention(q, k, v, 0.6, causal=True,
                                     blocks=[[int(j)] for j in order])
        _close(O, O_ref[0, 0], 1e-13, 1e-14, f"order {order}")
        _close(L, L_ref[0, 0], 1e-13, 1e-14, f"order {order} LSE")


# ---------------------------------------------------------------------------
# Special cases with closed forms
# ---------------------------------------------------------------------------

def pin_identical_keys(impl):
    """All keys equal: every visible logit of row i is scale*q_i.k0, so O_i is
    the (prefix) mean of V and LSE_i = scale*q_i.k0 + ln|J_i|."""
    rng = _rng(11)
    N, d = 9, 4
    q = _rand(rng, 1, 1, N, d)
    k0 = _rand(rng, d)
    k = np.broadcast_to(k0, (1, 1, N, d)).copy()
    v = _rand(rng, 1, 1, N, 3)
    sigma = float(np.float32(0.3))
    for causal in (False, True):
        O, L = impl.attention_ref(q, k, v, 0.3, causal=causal)
        for i in range(N):
            cnt = i + 1 if causal else N
            _close(O[0, 0, i], v[0, 0, :cnt].mean(axis=0), 1e-13, 1e-14, f"identical keys O[{i}]")
            want = sigma * float(q[0, 0, i] @ k0) + math.log(cnt)
            _close(L[0, 0, i], want, 1e-13, 1e-14, f"identical keys LSE[{i}]")


def pin_scale_zero(impl):
    """scale = 0: uniform weights, O = (prefix) mean of V, LSE = ln|J_i| exactly."""
    rng = _rng(12)
    N = 7
    q, k, v = _rand(rng, 2, 2, N, 3), _rand(rng, 2, 1, N, 3), _rand(rng, 2, 1, N, 2)
    for causal in (False, True):
        O, L = impl.attention_ref(q, k, v, 0.0, causal=causal)
        for b, h, i in itertools.product(range(2), range(2), range(N)):
            cnt = i + 1 if causal else N
            _close(O[b, h, i], v[b, 0, :cnt].mean(axis=0), 1e-14, 1e-15, "scale0 O")
            _close(L[b, h, i], math.log(cnt), 1e-15, 1e-15, "scale0 LSE")


def pin_dominant_logit(impl):
    """One key with logit 30 against zeros:
    O_i = (e^30 v_* + sum_{j != *} v_j) / (e^30 + |J_i| - 1) once the key is
    visible, the prefix mean before it; LSE_i = ln(e^30 + |J_i| - 1)."""
    rng = _rng(13)
    N, d, star = 8, 4, 3
    q = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 6.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, star, 0] = 10.0            # 0.5 * 6 * 10 = 30
    v = _rand(rng, 1, 1, N, 3)
    E30 = math.exp(30.0)
    for causal in (False, True):
        O, L = impl.attention_ref(q, k, v, 0.5, causal=causal)
        for i in range(N):
            vis = list(range(i + 1)) if causal else list(range(N))
            if star in vis:
                others = [j for j in vis if j != star]
                num = E30 * v[0, 0, star] + v[0, 0, others].sum(axis=0)
                den = E30 + len(others)
                _close(O[0, 0, i], num / den, 1e-13, 1e-15, f"dominant O[{i}]")
                _close(L[0, 0, i], math.log(den), 1e-14, 1e-15, f"dominant LSE[{i}]")
            else:
                _close(O[0, 0, i], v[0, 0, vis].mean(axis=0), 1e-13, 1e-15, f"dominant prefix O[{i}]")
                _close(L[0, 0, i], math.log(len(vis)), 1e-14, 1e-15, f"dominant prefix LSE[{i}]")


def pin_extreme_logits(impl):
    """One key with logit 900 against zeros (a spike far past fp64's exp
    range): rows that see it have O_i = v_* and LSE_i = 900 to fp64 accuracy,
    since e^-900 vanishes; rows that do not see it have the prefix mean.
    Exact in real arithmetic for any choice of stabiliser; fails any form that
    exponentiates a logit difference as large as 900.  The online recurrence is
    run with the spike in the first block and in the last."""
    rng = _rng(21)
    N, d, star = 6, 3, 2
    q = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 30.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, star, 0] = 30.0
    v = _rand(rng, 1, 1, N, 2)
    for causal in (False, True):
        O, L = impl.attention_ref(q, k, v, 1.0, causal=causal)
        rest = [j for j in range(N) if j != star]
        On, Ln = impl.online_attention(q[0, 0], k[0, 0], v[0, 0], 1.0, causal=causal,
                                       blocks=[[star], rest])
        Or, Lr = impl.online_attention(q[0, 0], k[0, 0], v[0, 0], 1.0, causal=causal,
                                       blocks=[rest, [star]])
        for i in range(N):
            vis = list(range(i + 1)) if causal else list(range(N))
            if star in vis:
                want_o, want_l = v[0, 0, star], 900.0
            else:
                want_o, want_l = v[0, 0, vis].mean(axis=0), math.log(len(vis))
            for tag, Oi, Li in (("ref", O[0, 0, i], L[0, 0, i]), ("online first", On[i], Ln[i]),
                                ("online last", Or[i], Lr[i])):
                _close(Oi, want_o, 1e-14, 1e-15, f"extreme {tag} O[{i}]")
                _close(Li, want_l, 1e-15, 1e-15, f"extreme {tag} LSE[{i}]")


def pin_rows_of_p_sum_to_one(impl):
    """With V = identity (N <= d), O = P: rows are >= 0, sum to 1, masked
    entries are exactly 0, and O agrees with attention_probs."""
    rng = _rng(14)
    N = 6
    q, k = _rand(rng, 1, 1, N, 5), _rand(rng, 1, 1, N, 5)
    v = np.eye(N)[None, None]
    for causal in (False, True):
        O, _ = impl.attention_ref(q, k, v, 1.3, causal=causal)
        P = impl.attention_probs(q[0, 0], k[0, 0], 1.3, causal=causal)
        assert (O >= 0).all(), "negative probability"
        _close(O[0, 0].sum(axis=1), np.ones(N), 1e-14, 0, "row sums")
        _close(O[0, 0], P, 1e-14, 1e-16, "O=P with V=I")
        _close(P.sum(axis=1), np.ones(N), 1e-14, 0, "attention_probs row sums")
        if causal:
            assert np.all(np.triu(O[0, 0], 1) == 0.0), "masked weight not exactly 0"


def pin_causal_first_and_last_rows(impl):
    """Causal row 0 sees only key 0: O_0 = v_0 exactly, LSE_0 = s_00.
    Causal row N-1 sees every key: it equals the non-causal row N-1."""
    rng = _rng(15)
    N = 10
    q, k, v = _rand(rng, 1, 2, N, 4), _rand(rng, 1, 2, N, 4), _rand(rng, 1, 2, N, 4)
    Oc, Lc = impl.attention_ref(q, k, v, 0.5, causal=True)
    On, Ln = impl.attention_ref(q, k, v, 0.5, causal=False)
    for h in range(2):
        assert np.array_equal(Oc[0, h, 0], v[0, h, 0]), "causal row 0 != v_0"
        _close(Lc[0, h, 0], 0.5 * float(q[0, h, 0] @ k[0, h, 0]), 1e-14, 1e-15, "LSE_0")
        _close(Oc[0, h, N - 1], On[0, h, N - 1], 1e-14, 1e-15, "last row")
        _close(Lc[0, h, N - 1], Ln[0, h, N - 1], 1e-14, 1e-15, "last row LSE")


def pin_gqa_equals_repeated_heads(impl):
    """GQA with groups of G equals MHA with each K/V head repeated G times in
    place (query head h reads K/V head h // G)."""
    rng = _rng(16)
    for Hq, Hkv in ((4, 2), (6, 3), (4, 1), (8, 2)):
        G = Hq // Hkv
        q = _rand(rng, 2, Hq, 5, 3)
        k, v = _rand(rng, 2, Hkv, 5, 3), _rand(rng, 2, Hkv, 5, 3)
        for causal in (False, True):
            O, L = impl.attention_ref(q, k, v, 0.4, causal=causal)
            O2, L2 = impl.attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                        0.4, causal=causal)
            _close(O, O2, 1e-15, 1e-16, f"GQA {Hq}/{Hkv}")
            _close(L, L2, 1e-15, 1e-16, f"GQA {Hq}/{Hkv} LSE")
            for h in range(Hq):
                assert impl.kv_head_of(h, Hq, Hkv) == h // G


def pin_permutations(impl):
    """Non-causal: permuting keys with their values leaves O and LSE unchanged;
    permuting queries permutes the output rows."""
    rng = _rng(17)
    N = 11
    q, k, v = _rand(rng, 1, 1, N, 4), _rand(rng, 1, 1, N, 4), _rand(rng, 1, 1, N, 4)
    O, L = impl.attention_ref(q, k, v, 0.7)
    pk = rng.permutation(N)
    O2, L2 = impl.attention_ref(q, k[:, :, pk], v[:, :, pk], 0.7)
    _close(O2, O, 1e-13, 1e-14, "key permutation")
    _close(L2, L, 1e-13, 1e-14, "key permutation LSE")
    pq = rng.permutation(N)
    O3, L3 = impl.attention_ref(q[:, :, pq], k, v, 0.7)
    _close(O3, O[:, :, pq], 1e-13, 1e-14, "query permutation")
    _close(L3, L[:, :, pq], 1e-13, 1e-14, "query permutation LSE")


def pin_key_shift(impl):
    """Adding u to every key shifts row i's logits by scale*q_i.u: O is
    unchanged and LSE_i moves by exactly that.  The shift is chosen to push
    logits past 700, where exp overflows fp64 unless the row maximum is
    subtracted first."""
    rng = _rng(18)
    N, d = 12, 4
    q = np.abs(_rand(rng, 1, 1, N, d)) + 0.5
    k, v = _rand(rng, 1, 1, N, d), _rand(rng, 1, 1, N, 3)
    u = np.full(d, 500.0)
    sigma = float(np.float32(0.75))
    for causal in (False, True):
        O, L = impl.attention_ref(q, k, v, 0.75, causal=causal)
        O2, L2 = impl.attention_ref(q, k + u, v, 0.75, causal=causal)
        _close(O2, O, 1e-9, 1e-10, "key shift O")
        _close(L2[0, 0], L[0, 0] + sigma * (q[0, 0] @ u), 1e-12, 1e-9, "key shift LSE")


def pin_row_subsets(impl):
    """Computing a subset of query rows gives those rows of the full result
    (the sampled checks of large workloads rely on this)."""
    rng = _rng(19)
    B, Hq, Hkv, N = 2, 4, 2, 37
    q, k, v = _rand(rng, B, Hq, N, 5), _rand(rng, B, Hkv, N, 5), _rand(rng, B, Hkv, N, 5)
    for causal in (False, True):
        O, L = impl.attention_ref(q, k, v, 0.45, causal=causal)
        r1 = np.array([0, 5, 36, 17])
        O1, L1 = impl.attention_ref(q, k, v, 0.45, causal=causal, rows=r1)
        _close(O1, O[:, :, r1], 1e-14, 1e-15, "rows 1-D")
        _close(L1, L[:, :, r1], 1e-14, 1e-15, "rows 1-D LSE")
        r3 = np.stack([np.stack([rng.choice(N, 6, replace=False) for _ in range(Hq)])
                       for _ in range(B)])
        O3, L3 = impl.attention_ref(q, k, v, 0.45, causal=causal, rows=r3, max_chunk_elems=80)
        for b, h in itertools.product(range(B), range(Hq)):
            _close(O3[b, h], O[b, h, r3[b, h]], 1e-14, 1e-15, "rows 3-D")
            _close(L3[b, h], L[b, h, r3[b, h]], 1e-14, 1e-15, "rows 3-D LSE")


def pin_torch_sdpa(impl):
    """Secondary: torch's CPU scaled_dot_product_attention in fp64 (the API the
    pages route through, [CANN-FA] section on calling from PyTorch)."""
    import torch
    rng = _rng(20)
    for Hq, Hkv, causal in ((4, 4, False), (4, 2, True), (6, 1, True)):
        q = _rand(rng, 2, Hq, 13, 8)
        k, v = _rand(rng, 2, Hkv, 13, 8), _rand(rng, 2, Hkv, 13, 8)
        O, _ = impl.attention_ref(q, k, v, 0.25, causal=causal)
        G = Hq // Hkv
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(np.repeat(k, G, axis=1))
        tv = torch.from_numpy(np.repeat(v, G, axis=1))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=0.25).numpy()
        _close(O, ref, 1e-12, 1e-13, f"sdpa {Hq}/{Hkv} causal={causal}")


def pin_decode_is_last_rows(impl):
    """A decode step equals the last Nq rows of full attention over the whole
    sequence (the queries placed at the last positions, any values in the
    other rows), causal or not, with GQA/MQA grouping."""
    rng = _rng(21)
    for B, Hq, Hkv, Nq, Nk in ((1, 1, 1, 1, 9), (2, 4, 2, 3, 17), (1, 6, 1, 5, 5), (2, 8, 2, 16, 40)):
        d = 6
        qd = _rand(rng, B, Hq, Nq, d)
        k, v = _rand(rng, B, Hkv, Nk, d), _rand(rng, B, Hkv, Nk, d)
        qfull = _rand(rng, B, Hq, Nk, d)
        qfull[:, :, Nk - Nq:] = qd
        rows = np.arange(Nk - Nq, Nk)
        for causal in (False, True):
            O, L = impl.attention_decode_ref(qd, k, v, 0.6, causal=causal)
            Of, Lf = impl.attention_ref(qfull, k, v, 0.6, causal=causal, rows=rows)
            _close(O, Of, 1e-13, 1e-14, f"decode vs last rows Nq={Nq} Nk={Nk} causal={causal}")
            _close(L, Lf, 1e-13, 1e-13, f"decode LSE vs last rows Nq={Nq} Nk={Nk} causal={causal}")


def pin_decode_brute_force(impl):
    """Decode against the textbook softmax in mpmath (no max subtraction)."""
    rng = _rng(22)
    for Hq, Hkv, Nq, Nk in ((1, 1, 1, 4), (2, 1, 2, 5), (4, 2, 3, 6)):
        q = _rand(rng, 1, Hq, Nq, 3)
        k, v = _rand(rng, 1, Hkv, Nk, 3), _rand(rng, 1, Hkv, Nk, 2)
        for causal in (False, True):
            O, L = impl.attention_decode_ref(q, k, v, 0.8, causal=causal)
            Ob, Lb = attention_brute(q, k, v, 0.8, causal=causal)
            _close(O, to_float_array(Ob), 1e-13, 1e-14, f"decode brute Nq={Nq} causal={causal}")
            _close(L, to_float_array(Lb), 1e-13, 1e-14, f"decode brute LSE Nq={Nq} causal={causal}")


def pin_decode_scale_zero_prefix_means(impl):
    """Scale 0: every visible logit is 0, so decode query i (position
    Nk - Nq + i) averages the values of keys 0 .. Nk - Nq + i and its LSE is
    ln(Nk - Nq + i + 1); non-causal, every query averages all Nk values."""
    rng = _rng(23)
    Nq, Nk = 4, 11
    q, k, v = _rand(rng, 1, 2, Nq, 5), _rand(rng, 1, 1, Nk, 5), _rand(rng, 1, 1, Nk, 5)
    O, L = impl.attention_decode_ref(q, k, v, 0.0, causal=True)
    for i in range(Nq):
        cnt = Nk - Nq + i + 1
        for h in range(2):
            _close(O[0, h, i], v[0, 0, :cnt].mean(axis=0), 1e-14, 1e-15, f"prefix mean row {i}")
            _close(L[0, h, i], np.log(cnt), 1e-15, 1e-15, f"ln count row {i}")
    O, L = impl.attention_decode_ref(q, k, v, 0.0, causal=False)
    _close(O[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (Nq, 5)), 1e-14, 1e-15, "non-causal mean")
    _close(L, np.full((1, 2, Nq), np.log(Nk)), 1e-15, 1e-15, "ln Nk")


def pin_decode_full_length(impl):
    """With Nq == Nk a decode step is ordinary attention."""
    rng = _rng(24)
    q, k, v = _rand(rng, 2, 4, 9, 5), _rand(rng, 2, 2, 9, 5), _rand(rng, 2, 2, 9, 5)
    for causal in (False, True):
        O, L = impl.attention_decode_ref(q, k, v, 0.3, causal=causal)
        Of, Lf = impl.attention_ref(q, k, v, 0.3, causal=causal)
        _close(O, Of, 1e-14, 1e-15, f"Nq == Nk causal={causal}")
        _close(L, Lf, 1e-14, 1e-15, f"Nq == Nk LSE causal={causal}")


ALL_PINS = [
    pin_golden_closed_forms,
    pin_scale_zero,
    pin_identical_keys,
    pin_dominant_logit,
    pin_extreme_logits,
    pin_rows_of_p_sum_to_one,
    pin_causal_first_and_last_rows,
    pin_gqa_equals_repeated_heads,
    pin_permutations,
    pin_key_shift,
    pin_row_subsets,
    pin_probs_brute_force,
    pin_online_equals_two_pass_exact,
    pin_online_block_invariance,
    pin_brute_force_small,
    pin_torch_sdpa,
    pin_decode_is_last_rows,
    pin_decode_brute_force,
    pin_decode_scale_zero_prefix_means,
    pin_decode_full_length,
]
