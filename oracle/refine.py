"""Double-precision oracle for stacked Sketch Attention refinement (test
infrastructure only: ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py`` may use it; the GPU library never does).

Follows section 3.3 (Stacked Refinement) of the SequenceO1 paper.  Layer l
takes the sketch Xt (Xt_0 = P, the k x d prototypes) and the user's history X
(n x d) and computes

    Q     = Xt Wq_l                       queries from the current sketch
    K     = X  Wk_l                       keys from the history
    Xhat  = softmax(Q K^T / sqrt(dh)) X   per head, values = X itself
    Xbar  = LN(Xt + Xhat)                 residual, layer norm
    Xt'   = LN(Xbar + FFN(Xbar))          SwiGLU FFN, residual, layer norm

with FFN(x) = (silu(x W1) * (x W3)) W2, inner width f (2d in the paper's
appendix G, "Sketch FFN").  Readings where the section is silent: heads
split the d channels into H blocks of dh (head h uses channels
[h dh, (h+1) dh) of Q, K and X, and writes those channels of Xhat); the
softmax runs over the history axis (the same reading as the single-layer
oracle; ``norm="prototype"`` gives the section 3.1 display instead); LN is
the usual per-row layer norm with a learned gain and bias and eps inside the
square root (default 1e-5); FFN matrices have no biases.  Every matrix is
stored [in, out] (y = x W), as the paper writes them.

Arithmetic: numpy float64 for the projections, the layer norms and the FFN;
the attention step is the pinned C oracle (``oracle.forward``), called once
per user with that user's queries, on exact double keys.  Inputs stored in
bf16 or fp32 are widened exactly.
"""
from __future__ import annotations

import numpy as np

from . import forward, widen64


def layer_norm(x, gain, bias, eps=1e-5):
    """Per-row layer norm over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gain, dtype=np.float64) + np.asarray(bias, dtype=np.float64)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_ffn(x, W1, W3, W2):
    """(silu(x W1) * (x W3)) W2, float64; W1, W3 [d, f], W2 [f, d]."""
    x = np.asarray(x, dtype=np.float64)
    return (silu(x @ widen64(W1)) * (x @ widen64(W3))) @ widen64(W2)


def attend(Q, X, Wk, cu_offsets, H, mask=None, norm="history", scale=None):
    """Xhat for every user: Q [B, k, d] (or [k, d] shared), X [rows, d]
    (the history, also the values), Wk [d, d].  Returns [B, k, d] float64."""
    Xd = widen64(X)
    Kd = Xd @ widen64(Wk)
    cu = np.asarray(cu_offsets, dtype=np.int64)
    B = len(cu) - 1
    d = Xd.shape[1]
    dh = d // H
    Q = np.asarray(Q, dtype=np.float64)
    k = Q.shape[-2]
    out = np.zeros((B, k, d), dtype=np.float64)
    mk = None if mask is None else np.asarray(mask)
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        Qb = Q if Q.ndim == 2 else Q[b]
        Pb = Qb.reshape(k, H, dh).transpose(1, 0, 2).copy()               # [H, k, dh]
        Kb = Kd[lo:hi].reshape(hi - lo, H, dh)
        Vb = Xd[lo:hi].reshape(hi - lo, H, dh)
        S, _ = forward(Pb, Kb, Vb, cu_offsets=np.array([0, hi - lo], dtype=np.int32),
                       mask=None if mk is None else mk[lo:hi], norm=norm, scale=scale)
        out[b] = S[0].transpose(1, 0, 2).reshape(k, d)
    return out


def refine(X, P0, layers, cu_offsets, H, mask=None, eps=1e-5, norm="history", scale=None, return_all=False):
    """Stacked refinement.  ``layers``: list of dicts with Wq, Wk [d, d],
    ln1_g, ln1_b, ln2_g, ln2_b [d], W1, W3 [d, f], W2 [f, d].  P0 [k, d].
    Returns the final sketch [B, k, d] (and every layer's sketch when
    ``return_all``)."""
    B = len(cu_offsets) - 1
    Xt = widen64(P0)
    sketches = []
    for L in layers:
        Q = Xt @ widen64(L["Wq"])
        Xhat = attend(Q, X, L["Wk"], cu_offsets, H, mask=mask, norm=norm, scale=scale)
        base = np.broadcast_to(Xt, Xhat.shape) if Xt.ndim == 2 else Xt
        Xbar = layer_norm(base + Xhat, widen64(L["ln1_g"]), widen64(L["ln1_b"]), eps)
        Xt = layer_norm(Xbar + swiglu_ffn(Xbar, L["W1"], L["W3"], L["W2"]), widen64(L["ln2_g"]),
                        widen64(L["ln2_b"]), eps)
        sketches.append(Xt)
    if B == 0:
        Xt = np.zeros((0,) + widen64(P0).shape, dtype=np.float64)
    return (Xt, sketches) if return_all else Xt
