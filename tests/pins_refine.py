"""Pins for the stacked-refinement oracle (``oracle/refine.py``): checks
against things other than that oracle.

Every pin takes the refinement module to check (the real one by default) so
that ``test_refine_oracle.py`` can run the same pins on mutated copies.

  brute_*     50-digit mpmath implementation of section 3.3 of the SequenceO1
              paper with materialised scores (``oracle.brute.refine``)
  library_*   torch's layer_norm and silu in float64
  closed_*    layer norm of a two-valued row; an FFN with W2 = 0; a user with
              one row (every prototype's attention output is that row)
  inv_*       rows of a layer-normed sketch have mean = bias and the gain's
              spread; permuting a user's rows; user isolation
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import brute
from oracle import refine as REFINE


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


def case(seed, d=4, H=2, k=3, f=8, lengths=(4, 1, 0, 4), n_layers=2, w_std=0.6):
    """Tiny random problem: X [rows, d], P0 [k, d], layers, cu."""
    rng = np.random.default_rng(seed)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    X = rng.standard_normal((int(cu[-1]), d))
    P0 = rng.standard_normal((k, d))
    layers = []
    for _ in range(n_layers):
        layers.append(dict(
            Wq=rng.standard_normal((d, d)) * w_std, Wk=rng.standard_normal((d, d)) * w_std,
            ln1_g=1 + 0.2 * rng.standard_normal(d), ln1_b=0.2 * rng.standard_normal(d),
            ln2_g=1 + 0.2 * rng.standard_normal(d), ln2_b=0.2 * rng.standard_normal(d),
            W1=rng.standard_normal((d, f)) * w_std, W3=rng.standard_normal((d, f)) * w_std,
            W2=rng.standard_normal((f, d)) * w_std))
    return X, P0, layers, cu, H


def _np(x):
    return np.array([[[float(v) for v in r] for r in u] for u in x], dtype=np.float64)


# ------------------------------------------------------------- brute force
def brute_two_layers(R=REFINE):
    X, P0, layers, cu, H = case(1)
    o = R.refine(X, P0, layers, cu, H)
    b = _np(brute.refine(X, P0, layers, cu, H))
    assert o.shape == b.shape and _rel(o, b) < 1e-12, _rel(o, b)


def brute_wider_heads_and_eps(R=REFINE):
    X, P0, layers, cu, H = case(2, d=6, H=3, k=2, f=5, lengths=(3, 5), n_layers=2, w_std=0.9)
    o = R.refine(X, P0, layers, cu, H, eps=1e-2)
    b = _np(brute.refine(X, P0, layers, cu, H, eps=1e-2))
    assert _rel(o, b) < 1e-12, _rel(o, b)


def brute_single_head(R=REFINE):
    X, P0, layers, cu, H = case(3, d=4, H=1, k=4, f=8, lengths=(6, 2), n_layers=1)
    o = R.refine(X, P0, layers, cu, H)
    b = _np(brute.refine(X, P0, layers, cu, H))
    assert _rel(o, b) < 1e-12, _rel(o, b)


# ---------------------------------------------------------- library routines
def library_layer_norm(R=REFINE):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 16)) * 3 + 1
    g, bta = rng.standard_normal(16), rng.standard_normal(16)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (16,), torch.from_numpy(g), torch.from_numpy(bta),
                                         eps=1e-5).numpy()
    assert _rel(R.layer_norm(x, g, bta, 1e-5), ref) < 1e-13


def library_silu(R=REFINE):
    x = np.linspace(-30, 30, 121)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(R.silu(x), ref, rtol=1e-14, atol=1e-300)


# -------------------------------------------------------------- closed forms
def closed_layer_norm_two_values(R=REFINE):
    # a row of a's and b's: mean (a+b)/2, variance ((a-b)/2)^2, so the
    # normalised row is +-(a-b)/2 / sqrt(((a-b)/2)^2 + eps)
    a, b, eps = 3.0, -1.0, 1e-3
    y = R.layer_norm(np.array([[a, b, a, b]]), np.ones(4), np.zeros(4), eps)
    v = 2.0 / np.sqrt(4.0 + eps)
    assert np.allclose(y, [[v, -v, v, -v]], rtol=1e-14)


def closed_ffn_zero_output(R=REFINE):
    x = np.random.default_rng(5).standard_normal((3, 4))
    W = np.random.default_rng(6).standard_normal((4, 8))
    assert np.array_equal(R.swiglu_ffn(x, W, W, np.zeros((8, 4))), np.zeros((3, 4)))
    # silu(0) = 0: a zero input gives zero whatever the weights
    assert np.array_equal(R.swiglu_ffn(np.zeros((2, 4)), W, W, W.T), np.zeros((2, 4)))
    # one hidden unit: silu(u) * v * w2 with u = x.w1 = 0.5 and v = x.w3 = 6
    x = np.array([[2.0, -2.0]])
    w1, w3, w2 = np.array([[0.5], [0.25]]), np.array([[2.0], [-1.0]]), np.array([[3.0, -2.0]])
    s = 0.5 / (1 + np.exp(-0.5)) * 6.0
    assert np.allclose(R.swiglu_ffn(x, w1, w3, w2), [[3 * s, -2 * s]], rtol=1e-14)


def closed_single_row_user(R=REFINE):
    # one history row x: every prototype's attention output is x itself
    # (whatever Wq and Wk), so one layer with gains 1, biases 0, eps 0 and
    # W2 = 0 gives LN(LN(P0 + x)) = the standardised rows of P0 + x
    d, k = 4, 3
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, d))
    P0 = rng.standard_normal((k, d))
    L = dict(Wq=rng.standard_normal((d, d)), Wk=rng.standard_normal((d, d)), ln1_g=np.ones(d), ln1_b=np.zeros(d),
             ln2_g=np.ones(d), ln2_b=np.zeros(d), W1=rng.standard_normal((d, 8)), W3=rng.standard_normal((d, 8)),
             W2=np.zeros((8, d)))
    out = R.refine(x, P0, [L], np.array([0, 1], dtype=np.int32), 2, eps=0.0)[0]
    y = P0 + x
    z = (y - y.mean(1, keepdims=True)) / y.std(1, keepdims=True)
    assert np.allclose(out, z, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariants
def inv_row_statistics(R=REFINE):
    X, P0, layers, cu, H = case(8, d=8, H=2, k=3, f=6, lengths=(5, 9))
    out = R.refine(X, P0, layers, cu, H, eps=0.0)
    g, bta = layers[-1]["ln2_g"], layers[-1]["ln2_b"]
    z = (out - bta) / g                         # the normalised rows before the affine part
    assert np.allclose(z.mean(-1), 0, atol=1e-12) and np.allclose((z ** 2).mean(-1), 1, atol=1e-12)


def inv_row_permutation(R=REFINE):
    X, P0, layers, cu, H = case(9, lengths=(6, 4))
    o = R.refine(X, P0, layers, cu, H)
    perm = np.concatenate([np.random.default_rng(9).permutation(6), 6 + np.arange(4)[::-1]])
    o2 = R.refine(X[perm], P0, layers, cu, H)
    assert _rel(o2, o) < 1e-13


def inv_user_isolation(R=REFINE):
    X, P0, layers, cu, H = case(10, lengths=(3, 4, 2))
    o = R.refine(X, P0, layers, cu, H)
    X2 = X.copy()
    X2[3:7] = -2 * X2[3:7]
    o2 = R.refine(X2, P0, layers, cu, H)
    assert np.array_equal(o[0], o2[0]) and np.array_equal(o[2], o2[2]) and not np.allclose(o[1], o2[1])


ALL_REFINE_PINS = [
    brute_two_layers, brute_wider_heads_and_eps, brute_single_head, library_layer_norm, library_silu,
    closed_layer_norm_two_values, closed_ffn_zero_output, closed_single_row_user, inv_row_statistics,
    inv_row_permutation, inv_user_isolation,
]
