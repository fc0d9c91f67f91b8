"""Plant plausible mistakes in copies of the oracle's C source and of its
Python layer (CPU only) and check that at least one pin rejects each copy.
This is what shows the pins are strong enough to trust the oracle: a dropped
term, a wrong sign, a wrong index or a transposed operand anywhere in it must
fail some pin."""
import os
import tempfile
import types

import pytest

import oracle
from pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "sa_oracle.c")
PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")

# (name, text in sa_oracle.c, replacement)
MUTANTS = [
    ("scale_dropped", "return acc * scale_of(pb);", "return acc;"),
    ("scale_squared", "1.0 / sqrt((double)pb->dh)", "1.0 / (double)pb->dh"),
    ("max_not_subtracted", "const double w = exp(s[t] - M);", "const double w = exp(s[t]);"),
    ("sign_flipped", "const double w = exp(s[t] - M);", "const double w = exp(M - s[t]);"),
    ("prototype_index_transposed", "((int64_t)h * pb->m + j) * pb->dh", "((int64_t)j * pb->H + h) * pb->dh"),
    ("value_head_offset_dropped", "const int64_t vbase = rows[t] * vstride(pb) + (int64_t)h * pb->dh;",
     "const int64_t vbase = rows[t] * vstride(pb);"),
    ("key_head_offset_dropped", "const int64_t kbase = row * kstride(pb) + (int64_t)h * pb->dh;",
     "const int64_t kbase = row * kstride(pb);"),
    ("normaliser_skips_first_row", "        Z += w;\n", "        if (t > 0) Z += w;\n"),
    ("not_normalised", "for (int e = 0; e < pb->dh; ++e) out[e] /= Z;", "(void)Z;"),
    ("user_rows_off_by_one", "*count = (int64_t)cu[b + 1] - cu[b];", "*count = (int64_t)cu[b + 1] - cu[b] - 1;"),
    ("mask_ignored", "if (mask && mask[row] == 0) continue;", "(void)mask;"),
    ("dense_lengths_ignored", "int64_t len = lengths ? lengths[b] : pb->L_max;", "int64_t len = pb->L_max;"),
    ("lse_missing_max", "*lse = M + log(Z);", "*lse = log(Z);"),
    ("bf16_widening_wrong", "<< 16;", "<< 15;"),
    ("prototype_axis_unnormalised", "const double a = exp(s[j] - M) / Z;", "const double a = exp(s[j] - M);"),
    ("prototype_axis_wrong_max", "            if (s[j] > M) M = s[j];\n        }\n        double Z = 0.0;\n        for (int j = 0; j < m; ++j) Z += exp(s[j] - M);",
     "        }\n        double Z = 0.0;\n        for (int j = 0; j < m; ++j) Z += exp(s[j] - M);"),
    ("value_used_as_key", "acc += widen(P, pb->in_dtype, pbase + e) * widen(K, pb->in_dtype, kbase + e);",
     "acc += widen(P, pb->in_dtype, pbase + e) * widen(K, pb->in_dtype, kbase + (pb->dh - 1 - e));"),
    ("per_user_prototypes_shared", "const int64_t pbase = (int64_t)b * pb->p_user_stride + ",
     "const int64_t pbase = "),
]

# Mistakes in the Python layer (oracle/__init__.py): the fused entry's
# projections and head split, and the per-user prototype stride.
PY_MUTANTS = [
    ("fused_head_split_transposed", "Vd.reshape(rows, H, dh)", "Vd.reshape(rows, dh, H).transpose(0, 2, 1)"),
    ("fused_values_x_are_keys", "Vd = project(X, Wv) if Wv is not None else _widen64(X)",
     "Vd = project(X, Wv) if Wv is not None else Kd"),
    ("fused_sample_x_head_offset", "_widen64(X)[rows, h * dh:(h + 1) * dh]", "_widen64(X)[rows, h:h + dh]"),
    ("fused_sample_keys_as_values", "Vd = project(X, Wv, rows=rows, c0=h * dh, nc=dh) if Wv is not None",
     "Vd = Kd if Wv is not None"),
    ("per_user_stride_ignored", "return int(Pr.shape[1] * Pr.shape[2] * Pr.shape[3])", "return 0"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mutant.c")
        with open(path, "w") as f:
            f.write(mutated)
        lib = oracle.build(extra_flags=("-w",), out=os.path.join(td, "libmutant.so"), src=path)
        failed = []
        with oracle.using(lib):
            for pin in ALL_PINS:
                try:
                    pin()
                except Exception as e:  # AssertionError, or a crash-free error path
                    failed.append((pin.__name__, type(e).__name__))
        assert failed, f"no pin rejects the mutant '{name}'"


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(name, old, new, monkeypatch):
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = PY_SRC
    exec(compile(src.replace(old, new, 1), PY_SRC, "exec"), mod.__dict__)
    for fn in ("forward", "forward_sample", "assignment", "project", "fused_forward", "fused_forward_sample",
               "_user_stride"):
        monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"no pin rejects the mutant '{name}'"


def test_python_copy_unmutated_passes_every_pin(monkeypatch):
    """Control for the Python mutants: the same loading mechanism with no
    mistake planted passes every pin, so the mutants above fail for their
    mistake and not for the way they are loaded."""
    mod = types.ModuleType("oracle_copy")
    mod.__file__ = PY_SRC
    exec(compile(open(PY_SRC).read(), PY_SRC, "exec"), mod.__dict__)
    for fn in ("forward", "forward_sample", "assignment", "project", "fused_forward", "fused_forward_sample",
               "_user_stride"):
        monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    for pin in ALL_PINS:
        pin()
