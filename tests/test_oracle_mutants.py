"""Mutation test of the oracle's pins.

Each mutant plants one plausible mistake (a dropped term, a wrong sign, a
wrong index or axis, a transposed or swapped operand, an off-by-one mask) into
a copy of the oracle's source, on the CPU, and checks that at least one pin
rejects it.  This is what makes the pins evidence: a pin set that passed a
broken oracle would prove nothing.
"""

import inspect
import types

import pytest

import oracle.attention as oracle_impl
from oracle_pins import ALL_PINS

SOURCE = inspect.getsource(oracle_impl)

MUTANTS = {
    # attention_ref (the two-pass oracle every GPU result is compared with)
    "scale_dropped": ("S = sigma * (Qc @ K.T)", "S = (Qc @ K.T)"),
    "scale_squared": ("S = sigma * (Qc @ K.T)", "S = sigma * sigma * (Qc @ K.T)"),
    "logits_transposed": ("S = sigma * (Qc @ K.T)", "S = sigma * (K @ Qc.T)[:len(ri)][:, :len(ri)].T"),
    "causal_strict": ("S = np.where(keys <= ri[:, None], S, -np.inf)",
                      "S = np.where(keys < ri[:, None], S, -np.inf)"),
    "causal_one_ahead": ("S = np.where(keys <= ri[:, None], S, -np.inf)",
                         "S = np.where(keys <= ri[:, None] + 1, S, -np.inf)"),
    "causal_reversed": ("S = np.where(keys <= ri[:, None], S, -np.inf)",
                        "S = np.where(keys >= ri[:, None], S, -np.inf)"),
    "no_max_subtraction": ("                E = np.exp(S - m[:, None])\n                l = E.sum(axis=1)\n                P = E / l[:, None]",
                           "                E = np.exp(S)\n                l = E.sum(axis=1)\n                P = E / l[:, None]"),
    "exp_sign": ("                E = np.exp(S - m[:, None])\n                l = E.sum(axis=1)\n                P = E / l[:, None]",
                 "                E = np.exp(m[:, None] - S)\n                l = E.sum(axis=1)\n                P = E / l[:, None]"),
    "max_wrong_axis": ("                m = S.max(axis=1)\n                E",
                       "                m = S.max(axis=0)[:len(ri)]\n                E"),
    "min_instead_of_max": ("                m = S.max(axis=1)\n                E",
                           "                m = np.where(np.isinf(S), np.inf, S).min(axis=1)\n                E"),
    "no_normalisation": ("                P = E / l[:, None]\n                O[b",
                         "                P = E\n                O[b"),
    "normalise_by_max_term": ("                P = E / l[:, None]\n                O[b",
                              "                P = E / E.max(axis=1)[:, None]\n                O[b"),
    "values_from_keys": ("O[b, hq, c0:c0 + len(ri)] = P @ V", "O[b, hq, c0:c0 + len(ri)] = P @ K"),
    "lse_missing_max": ("LSE[b, hq, c0:c0 + len(ri)] = m + np.log(l)",
                        "LSE[b, hq, c0:c0 + len(ri)] = np.log(l)"),
    "lse_log_sign": ("LSE[b, hq, c0:c0 + len(ri)] = m + np.log(l)",
                     "LSE[b, hq, c0:c0 + len(ri)] = m - np.log(l)"),
    "gqa_modulo": ("    return hq // group", "    return hq % Hkv"),
    "gqa_interleaved": ("    return hq // group", "    return (hq * Hkv) % Hkv + hq % Hkv"),
    "rows_ignored": ("Qc = q[b, hq, ri].astype(np.float64)",
                     "Qc = q[b, hq, np.arange(len(ri))].astype(np.float64)"),
    # attention_probs
    "probs_causal_strict": ("S = np.where(j <= i, S, -np.inf)", "S = np.where(j < i, S, -np.inf)"),
    "probs_unnormalised": ("    return E / l[:, None]              #", "    return E                           #"),
    "probs_sum_wrong_axis": ("    l = E.sum(axis=1)                  #", "    l = E.sum(axis=0)                  #"),
    # online_attention (the pages' recurrence, used to pin the two-pass form)
    "online_corr_sign": ("corr = exp(m - m_new)", "corr = exp(m_new - m) if m > float('-inf') else 0 * m_new"),
    "online_drop_corr_in_l": ("l_new = l * corr + sum(e)", "l_new = l + sum(e)"),
    "online_keep_drops_l": ("keep = l * corr / l_new", "keep = corr / l_new"),
    "online_keep_drops_corr": ("keep = l * corr / l_new", "keep = l / l_new"),
    "online_deferred_no_rescale": ("o = [o[c] * corr + sum(", "o = [o[c] + sum("),
    "online_causal_strict": ("js = [j for j in blk if (not causal) or j <= i]",
                             "js = [j for j in blk if (not causal) or j < i]"),
    "online_lse_no_max": ("L_out.append(m + log(l))", "L_out.append(log(l))"),
    "online_max_ignores_old": ("m_new = max([m] + s)", "m_new = max(s)"),
    # attention_decode_ref
    "decode_no_offset": ("    pos = (Nk - Nq) + np.arange(Nq)", "    pos = np.arange(Nq)"),
    "decode_offset_off_by_one": ("    pos = (Nk - Nq) + np.arange(Nq)", "    pos = (Nk - Nq - 1) + np.arange(Nq)"),
    "decode_mask_strict": ("S = np.where(keys[None, :] <= pos[:, None], S, -np.inf)",
                           "S = np.where(keys[None, :] < pos[:, None], S, -np.inf)"),
    "decode_first_positions": ("S = np.where(keys[None, :] <= pos[:, None], S, -np.inf)",
                               "S = np.where(keys[None, :] <= pos[:, None] - (Nk - Nq), S, -np.inf)"),
    "decode_unnormalised": ("            O[b, hq] = (E / l[:, None]) @ V", "            O[b, hq] = E @ V"),
    "decode_lse_no_max": ("            LSE[b, hq] = m + np.log(l)", "            LSE[b, hq] = np.log(l)"),
    "decode_wrong_head": ("V = v[b, kvh].astype(np.float64)\n            S = sigma * (q[b, hq]",
                          "V = v[b, hq % Hkv].astype(np.float64)\n            S = sigma * (q[b, hq]"),
}


def _mutant_module(name, old, new):
    assert SOURCE.count(old) == 1, f"mutant {name}: pattern found {SOURCE.count(old)} times"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__dict__["__name__"] = mod.__name__
    exec(compile(SOURCE.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_rejects_mutant(name):
    old, new = MUTANTS[name]
    mod = _mutant_module(name, old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            with __import__("warnings").catch_warnings():
                __import__("warnings").simplefilter("ignore")
                __import__("numpy").seterr(all="ignore")
                pin(mod)
        except Exception as exc:  # AssertionError, or a crash caused by the mistake
            caught.append((pin.__name__, type(exc).__name__))
            break
        finally:
            __import__("numpy").seterr(all="warn")
    assert caught, f"no pin rejects mutant {name}"


def test_unmutated_source_passes_all_pins():
    mod = _mutant_module("identity", "def kv_head_of", "def kv_head_of")
    for pin in ALL_PINS:
        pin(mod)
