"""The backward oracle against its pins, and mutated copies of it against
the same pins (each plausible mistake must fail at least one).  CPU only."""
import types

import numpy as np
import pytest

import oracle
from oracle import backward as BACKWARD
from pins_backward import ALL_BACKWARD_PINS

SRC = BACKWARD.__file__

# (name, text in oracle/backward.py, replacement)
MUTANTS = [
    ("softmax_correction_dropped", "ds = A * (dA - (A * dA).sum(axis=1, keepdims=True))", "ds = A * dA"),
    ("correction_over_wrong_axis", "ds = A * (dA - (A * dA).sum(axis=1, keepdims=True))",
     "ds = A * (dA - (A * dA).sum(axis=0, keepdims=True))"),
    ("scale_missing_in_dK", "dK[rows, h] += c * (ds.T @ Pj)", "dK[rows, h] += ds.T @ Pj"),
    ("scale_missing_in_dP", "dP[h] += c * (ds @ Kb)", "dP[h] += ds @ Kb"),
    ("dK_sign_flipped", "dK[rows, h] += c * (ds.T @ Pj)", "dK[rows, h] -= c * (ds.T @ Pj)"),
    ("dV_prototypes_misindexed", "dV[rows, h] += A.T @ G", "dV[rows, h] += A.T @ G[::-1]"),
    ("dA_uses_keys", "dA = G @ Vb.T", "dA = G @ Kb.T"),
    ("softmax_over_prototypes", "A /= A.sum(axis=1, keepdims=True)", "A /= A.sum(axis=0, keepdims=True)"),
    ("mask_ignored", "        rows = rows[np.asarray(mask).reshape(-1)[rows] != 0]\n", "        pass\n"),
    ("per_user_dP_into_first_user", "dP[b, h] += c * (ds @ Kb)", "dP[0, h] += c * (ds @ Kb)"),
    ("dense_lengths_ignored", "n = L_max if lengths is None else max(0, min(int(lengths[b]), L_max))", "n = L_max"),
    ("scale_default_wrong", "c = 1.0 / np.sqrt(dh) if scale is None else float(scale)",
     "c = 1.0 / dh if scale is None else float(scale)"),
]


@pytest.mark.parametrize("pin", ALL_BACKWARD_PINS, ids=[p.__name__ for p in ALL_BACKWARD_PINS])
def test_backward_pin(pin):
    pin()


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new).replace("from . import widen64", "")
    mod = types.ModuleType("backward_mutant")
    mod.__dict__.update(widen64=oracle.widen64)
    exec(compile(src, "backward_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_is_caught(name, old, new):
    R = _mutant(old, new)
    caught = []
    for pin in ALL_BACKWARD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(R)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant {name}"
