"""The STCA oracle against its pins, and mutated copies of it against the
same pins (each plausible mistake must fail at least one).  CPU only."""
import types

import numpy as np
import pytest

import oracle
from oracle import stca as STCA
from pins_stca import ALL_STCA_PINS

SRC = STCA.__file__

# (name, text in oracle/stca.py, replacement)
MUTANTS = [
    ("scale_uses_model_width", "c = 1.0 / np.sqrt(dh)", "c = 1.0 / np.sqrt(D)"),
    ("query_not_projected", "q = xt[t] @ Wq", "q = xt[t]"),
    ("keys_not_folded_in", "u = q[cols] @ Wk[:, cols].T", "u = q"),
    ("key_matrix_not_transposed", "u = q[cols] @ Wk[:, cols].T", "u = q[cols] @ Wk[cols, :]"),
    ("heads_share_first_block", "u = q[cols] @", "u = q[:dh] @"),
    ("weights_not_normalised", "a /= a.sum()", "pass"),
    ("values_through_keys", "out[t, cols] = y @ Wv[:, cols]", "out[t, cols] = y @ Wk[:, cols]"),
    ("value_columns_not_head", "out[t, cols] = y @ Wv[:, cols]", "out[t, cols] = y @ Wv[:, :dh]"),
    ("window_ignored", "Xw = rows[lo:hi]", "Xw = rows"),
    ("window_drops_last_row", "Xw = rows[lo:hi]", "Xw = rows[lo:max(lo, hi - 1)]"),
    ("weights_from_keys_not_rows", "y = a @ Xw", "y = a @ (Xw @ Wk)"),
]


@pytest.mark.parametrize("pin", ALL_STCA_PINS, ids=[p.__name__ for p in ALL_STCA_PINS])
def test_stca_pin(pin):
    pin()


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new).replace("from . import widen64", "")
    mod = types.ModuleType("stca_mutant")
    mod.__dict__.update(widen64=oracle.widen64)
    exec(compile(src, "stca_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_stca_mutant_is_caught(name, old, new):
    R = _mutant(old, new)
    caught = []
    for pin in ALL_STCA_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(R)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant {name}"
