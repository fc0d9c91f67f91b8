"""Pins for the STCA oracle (``oracle/stca.py``): checks against things other
than that oracle.  Every pin takes the module to check (the real one by
default), so ``test_stca_oracle.py`` runs them on mutated copies.

  brute_*     50-digit mpmath evaluation of section 2.3's attention as written
              (keys and values projected, no reordering: ``oracle.brute.stca``)
  library_*   torch's scaled_dot_product_attention in float64 on the same
              un-reordered form, windows as a boolean attention mask
  closed_*    a window of one row (the weight is 1, so the output is that row
              through W_V); W_Q = 0 (uniform weights: the window's mean row
              through W_V); empty windows and targets outside every user give 0
  inv_*       a window equals slicing the history; permuting rows; targets
              and users do not interact; linearity in W_V
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import brute
from oracle import stca as STCA


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


def case(seed, D=4, h=2, lengths=(5, 1, 0, 6), targets=(2, 1, 1, 3), w_std=0.7, windows=False):
    """Tiny random problem: xt [T, D], X [rows, D], Wq, Wk, Wv [D, D], cu, tcu
    and optional windows [T, 2] (relative to the user's first row)."""
    rng = np.random.default_rng(seed)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    tcu = np.zeros(len(targets) + 1, dtype=np.int32)
    tcu[1:] = np.cumsum(targets)
    T = int(tcu[-1])
    xt = rng.standard_normal((T, D))
    X = rng.standard_normal((int(cu[-1]), D))
    Wq, Wk, Wv = (rng.standard_normal((D, D)) * w_std for _ in range(3))
    win = None
    if windows:
        win = np.zeros((T, 2), dtype=np.int32)
        for b, n in enumerate(lengths):
            for t in range(int(tcu[b]), int(tcu[b + 1])):
                lo = int(rng.integers(0, n + 1))
                win[t] = (lo, int(rng.integers(lo, n + 1)) if n else 0)
    return dict(xt=xt, X=X, Wq=Wq, Wk=Wk, Wv=Wv, cu=cu, tcu=tcu, h=h, windows=win)


def _run(R, c, **over):
    a = dict(c, **over)
    return R.stca_attention(a["xt"], a["X"], a["Wq"], a["Wk"], a["Wv"], a["cu"], a["tcu"], a["h"],
                            windows=a["windows"])


def _np(x):
    return np.array([[float(v) for v in r] for r in x], dtype=np.float64)


# ------------------------------------------------------------- brute force
def brute_plain(R=STCA):
    c = case(1)
    o = _run(R, c)
    b = _np(brute.stca(c["xt"], c["X"], c["Wq"], c["Wk"], c["Wv"], c["cu"], c["tcu"], c["h"]))
    assert _rel(o, b) < 1e-12, _rel(o, b)


def brute_windows_three_heads(R=STCA):
    c = case(2, D=6, h=3, lengths=(4, 7), targets=(3, 2), windows=True)
    o = _run(R, c)
    b = _np(brute.stca(c["xt"], c["X"], c["Wq"], c["Wk"], c["Wv"], c["cu"], c["tcu"], c["h"], c["windows"]))
    assert _rel(o, b) < 1e-12, _rel(o, b)


# ----------------------------------------------------------- library routine
def library_sdpa(R=STCA):
    """torch's attention on the section 2.3 form (keys and values projected)."""
    c = case(3, D=32, h=4, lengths=(37, 12, 25), targets=(5, 2, 4), w_std=0.25, windows=True)
    o = _run(R, c)
    D, h = 32, 4
    dh = D // h
    xt, X = torch.from_numpy(c["xt"]), torch.from_numpy(c["X"])
    Wq, Wk, Wv = (torch.from_numpy(c[k]) for k in ("Wq", "Wk", "Wv"))
    ref = np.zeros_like(o)
    nonempty = np.zeros(len(o), dtype=bool)
    for b in range(3):
        r0, r1 = int(c["cu"][b]), int(c["cu"][b + 1])
        t0, t1 = int(c["tcu"][b]), int(c["tcu"][b + 1])
        n = r1 - r0
        mask = torch.zeros((t1 - t0, n), dtype=torch.bool)
        for t in range(t0, t1):
            lo, hi = (int(v) for v in c["windows"][t])
            mask[t - t0, lo:hi] = True
            nonempty[t] = hi > lo
        for hh in range(h):
            cs = slice(hh * dh, (hh + 1) * dh)
            q = (xt[t0:t1] @ Wq)[:, cs]
            k = (X[r0:r1] @ Wk)[:, cs]
            v = (X[r0:r1] @ Wv)[:, cs]
            att = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None],
                                                                   attn_mask=mask[None])[0]
            ref[t0:t1, cs] = att.numpy()
    assert nonempty.sum() >= 6
    assert _rel(o[nonempty], ref[nonempty]) < 1e-12, _rel(o[nonempty], ref[nonempty])
    assert np.all(o[~nonempty] == 0)


# -------------------------------------------------------------- closed forms
def closed_single_row_window(R=STCA):
    c = case(4, D=8, h=2, lengths=(6,), targets=(3,))
    c["windows"] = np.array([[2, 3], [5, 6], [0, 1]], dtype=np.int32)
    o = _run(R, c)
    for t, i in enumerate((2, 5, 0)):
        assert np.allclose(o[t], c["X"][i] @ c["Wv"], rtol=1e-13, atol=1e-13)


def closed_zero_query_weights(R=STCA):
    # W_Q = 0: every score is 0, the weights are uniform over the window
    c = case(5, D=8, h=4, lengths=(9, 4), targets=(2, 2), windows=True)
    c["Wq"] = np.zeros((8, 8))
    o = _run(R, c)
    for b in range(2):
        r0 = int(c["cu"][b])
        for t in range(int(c["tcu"][b]), int(c["tcu"][b + 1])):
            lo, hi = (int(v) for v in c["windows"][t])
            want = c["X"][r0 + lo:r0 + hi].mean(axis=0) @ c["Wv"] if hi > lo else np.zeros(8)
            assert np.allclose(o[t], want, rtol=1e-13, atol=1e-13)


def closed_empty_and_orphan_targets(R=STCA):
    c = case(6, D=4, h=2, lengths=(3, 0), targets=(1, 2))
    c["tcu"] = np.array([0, 1, 3], dtype=np.int32)
    xt = np.concatenate([c["xt"], np.ones((2, 4))])          # targets 3, 4 belong to no user
    o = _run(R, c, xt=xt)
    assert np.all(o[1:] == 0) and np.any(o[0] != 0)
    c["windows"] = np.array([[2, 2], [0, 0], [0, 0], [0, 0], [0, 0]], dtype=np.int32)
    assert np.all(_run(R, c, xt=xt) == 0)


# ---------------------------------------------------------------- invariants
def inv_window_is_slicing(R=STCA):
    c = case(7, D=8, h=2, lengths=(11,), targets=(4,))
    c["windows"] = np.array([[3, 9], [0, 11], [10, 11], [4, 5]], dtype=np.int32)
    o = _run(R, c)
    for t in range(4):
        lo, hi = (int(v) for v in c["windows"][t])
        s = _run(R, c, xt=c["xt"][t:t + 1], X=c["X"][lo:hi], cu=np.array([0, hi - lo], dtype=np.int32),
                 tcu=np.array([0, 1], dtype=np.int32), windows=None)
        assert _rel(s[0], o[t]) < 1e-14


def inv_row_permutation(R=STCA):
    c = case(8, D=8, h=2, lengths=(9, 5), targets=(3, 2))
    o = _run(R, c)
    perm = np.concatenate([np.random.default_rng(8).permutation(9), 9 + np.arange(5)[::-1]])
    assert _rel(_run(R, c, X=c["X"][perm]), o) < 1e-13


def inv_isolation(R=STCA):
    c = case(9, D=8, h=4, lengths=(4, 6, 3), targets=(2, 3, 1))
    o = _run(R, c)
    X2 = c["X"].copy()
    X2[4:10] = -3 * X2[4:10]
    o2 = _run(R, c, X=X2)
    assert np.array_equal(o[:2], o2[:2]) and np.array_equal(o[5:], o2[5:]) and not np.allclose(o[2:5], o2[2:5])
    # targets of a user are independent: reversing them reverses the outputs
    xt = c["xt"].copy()
    xt[2:5] = xt[2:5][::-1]
    o3 = _run(R, c, xt=xt)
    assert np.array_equal(o3[2:5], o[2:5][::-1])


def inv_linear_in_values(R=STCA):
    c = case(10, D=8, h=2, lengths=(7,), targets=(3,))
    W2 = np.random.default_rng(10).standard_normal((8, 8))
    a = _run(R, c)
    b = _run(R, c, Wv=W2)
    ab = _run(R, c, Wv=2.0 * c["Wv"] - 0.5 * W2)
    assert np.allclose(ab, 2.0 * a - 0.5 * b, rtol=1e-12, atol=1e-12)


ALL_STCA_PINS = [
    brute_plain, brute_windows_three_heads, library_sdpa, closed_single_row_window, closed_zero_query_weights,
    closed_empty_and_orphan_targets, inv_window_is_slicing, inv_row_permutation, inv_isolation,
    inv_linear_in_values,
]
