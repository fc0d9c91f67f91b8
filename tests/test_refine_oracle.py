"""The stacked-refinement oracle against its pins, and mutated copies of it
against the same pins (each plausible mistake must fail at least one).  CPU
only."""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import refine as REFINE
from pins_refine import ALL_REFINE_PINS

SRC = REFINE.__file__

# (name, text in oracle/refine.py, replacement)
MUTANTS = [
    ("ln_mean_not_subtracted", "return (x - mu) / np.sqrt(var + eps)", "return x / np.sqrt(var + eps)"),
    ("ln_eps_outside_sqrt", "np.sqrt(var + eps)", "(np.sqrt(var) + eps)"),
    ("ln_bias_dropped", "* np.asarray(gain, dtype=np.float64) + np.asarray(bias, dtype=np.float64)",
     "* np.asarray(gain, dtype=np.float64)"),
    ("silu_is_sigmoid", "return x / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(-x))"),
    ("gate_swapped", "silu(x @ widen64(W1)) * (x @ widen64(W3))", "silu(x @ widen64(W3)) * (x @ widen64(W1))"),
    ("keys_not_projected", "Kd = Xd @ widen64(Wk)", "Kd = Xd"),
    ("queries_not_projected", 'Q = Xt @ widen64(L["Wq"])', "Q = Xt"),
    ("heads_blocked_wrongly", "Pb = Qb.reshape(k, H, dh).transpose(1, 0, 2).copy()", "Pb = Qb.reshape(H, k, dh).copy()"),
    ("first_residual_dropped", "layer_norm(base + Xhat,", "layer_norm(Xhat,"),
    ("second_residual_dropped", "layer_norm(Xbar + swiglu_ffn(", "layer_norm(0 * Xbar + swiglu_ffn("),
    ("layer_norms_swapped", 'widen64(L["ln1_g"]), widen64(L["ln1_b"])', 'widen64(L["ln2_g"]), widen64(L["ln2_b"])'),
    ("values_are_keys", "Vb = Xd[lo:hi].reshape(hi - lo, H, dh)", "Vb = Kd[lo:hi].reshape(hi - lo, H, dh)"),
]


@pytest.mark.parametrize("pin", ALL_REFINE_PINS, ids=[p.__name__ for p in ALL_REFINE_PINS])
def test_refine_pin(pin):
    pin()


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new).replace("from . import forward, widen64", "")
    mod = types.ModuleType("refine_mutant")
    mod.__dict__.update(forward=oracle.forward, widen64=oracle.widen64)
    exec(compile(src, "refine_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_refine_mutant_is_caught(name, old, new):
    R = _mutant(old, new)
    caught = []
    for pin in ALL_REFINE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(R)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant {name}"
