"""The backward oracle against its pins, and planted mistakes that some pin
must reject (CPU only)."""

import os
import types
import warnings

import numpy as np
import pytest

import oracle.backward as backward
from oracle_bwd_pins import BWD_PINS

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = open(os.path.join(HERE, "..", "oracle", "backward.py")).read()


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_backward_oracle_pin(pin):
    pin(backward)


MUTANTS = {
    "dv_untransposed": ("dv[b, kvh] += P.T @ dO", "dv[b, kvh] += P @ dO"),
    "dp_with_k": ("dP = dO @ V.T", "dP = dO @ K.T"),
    "ds_no_delta": ("dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dS = P * dP"),
    "ds_delta_wrong_axis": ("(P * dP).sum(axis=1, keepdims=True)", "(P * dP).sum(axis=0, keepdims=True)"),
    "dq_no_scale": ("dq[b, hq] = sigma * (dS @ K)", "dq[b, hq] = (dS @ K)"),
    "dk_untransposed": ("dk[b, kvh] += sigma * (dS.T @ Q)", "dk[b, kvh] += sigma * (dS @ Q)"),
    "dk_overwritten": ("dk[b, kvh] += sigma * (dS.T @ Q)", "dk[b, kvh] = sigma * (dS.T @ Q)"),
    "dv_overwritten": ("dv[b, kvh] += P.T @ dO", "dv[b, kvh] = P.T @ dO"),
    "wrong_head": ("kvh = kv_head_of(hq, Hq, Hkv)", "kvh = hq % Hkv"),
    "no_causal_in_p": ("P = attention_probs(Q, K, scale, causal=causal)", "P = attention_probs(Q, K, scale)"),
    "delta_uses_do_twice": ("(np.asarray(o).astype(np.float64) * np.asarray(do).astype(np.float64))",
                            "(np.asarray(do).astype(np.float64) * np.asarray(do).astype(np.float64))"),
}


def _mutant(name, old, new):
    assert SOURCE.count(old) == 1, f"mutant {name}: pattern found {SOURCE.count(old)} times"
    src = SOURCE.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"oracle_backward_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_rejects_backward_mutant(name):
    mod = _mutant(name, *MUTANTS[name])
    caught = None
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        old = np.seterr(all="ignore")
        try:
            for pin in BWD_PINS:
                try:
                    pin(mod)
                except Exception as exc:  # AssertionError, or a crash caused by the mistake
                    caught = (pin.__name__, type(exc).__name__)
                    break
        finally:
            np.seterr(**old)
    assert caught, f"no pin rejects mutant {name}"


def test_unmutated_backward_passes_through_the_mutant_loader():
    mod = _mutant("identity", "def attention_bwd_delta", "def attention_bwd_delta")
    for pin in BWD_PINS:
        pin(mod)
