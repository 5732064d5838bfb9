"""The fp64 backward oracle against its pins, and broken copies of it
against the same pins (each plausible mistake must fail at least one)."""
import os
import types

import numpy as np
import pytest

import oracle
import oracle.backward
from oracle_bwd_pins import ALL_BWD_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(oracle.backward.attention_backward)


MUTANTS = {
    "no_softmax_jacobian_term": ("dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))", "dS = P * dP"),
    "jacobian_column_sum": ("np.sum(P * dP, axis=1, keepdims=True)", "np.sum(P * dP, axis=0, keepdims=True)"),
    "dv_untransposed": ("dV = P.T @ dO", "dV = P @ dO"),
    "dq_without_scale": ("dQ = scale * (dS @ K)", "dQ = dS @ K"),
    "dk_untransposed": ("dK = scale * (dS.T @ Q)", "dK = scale * (dS @ Q)"),
    "dk_uses_keys": ("dK = scale * (dS.T @ Q)", "dK = scale * (dS.T @ K)"),
    "dp_uses_keys": ("dP = dO @ V.T", "dP = dO @ K.T"),
    "no_causal_mask": ("    if causal:\n        S = np.where", "    if False:\n        S = np.where"),
    "upper_triangle": ("np.tril(np.ones((n, n), dtype=bool))", "np.triu(np.ones((n, n), dtype=bool))"),
    "scores_scale_squared": ("S = (Q @ K.T) * scale", "S = (Q @ K.T) * scale * scale"),
    "dv_from_scores": ("dV = P.T @ dO", "dV = E.T @ dO"),
    "packed_first_token": ("t0, t1 = int(cu[b]), int(cu[b + 1])", "t0, t1 = 0, int(cu[b + 1]) - int(cu[b])"),
}


def _mutant_module(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = src.replace(old, new).replace("from . import _widen", "")
    mod = types.ModuleType(f"bwd_mutant_{name}")
    mod.__dict__["_widen"] = oracle._widen
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name):
    mod = _mutant_module(name)
    caught = []
    for pin in ALL_BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod.attention_backward)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every backward pin"
