"""Double-precision oracle for STCA single-query target-to-history cross
attention with the reordering of the SequenceO1 paper's appendix G.2.1 (test
infrastructure only: ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py`` may use it; the GPU library never does).

Section 2.3 ("STCA Recap") defines one attention of a target vector q over a
history X [L, D] as softmax((q W_Q)(X W_K)^T / sqrt(dh)) (X W_V), with h heads
of width dh = D / h.  Appendix G.2.1 evaluates it without the L x dh key and
value projections: per head (channels c = [hh dh, (hh+1) dh) of the
projections),

    u     = (q W_Q[:, c]) W_K[:, c]^T        [D]   (query folded into key space)
    alpha = softmax(u X^T / sqrt(dh))        [L]   over the target's rows
    y     = alpha X                          [D]
    o[c]  = y W_V[:, c]                      [dh]

and the target's output is the h blocks o[c] side by side, [D].  This module
takes those steps in that order, one target and one head at a time, in numpy
float64 (inputs stored in bf16 or fp32 are widened exactly).

Readings where the pages are silent: targets are grouped by user (the
multi-request batching of section 4.2 serves many targets of one user
together), user b's history rows are X[cu[b]:cu[b+1]] and its targets are
t_offsets[b]..t_offsets[b+1]-1; the request-aware masking of section 4.2 is a
per-target window [lo, hi) of the user's rows (relative to the user's first
row, clipped to the user) outside which a target's weights are zero; a target
with no row in its window, and a target outside every user, gets 0; matrices
are stored [in, out] (y = x W) as the paper writes them.  The output
projection W_O and the query-side FFN that follow in a full STCA layer are
one-token transforms outside this attention.
"""
from __future__ import annotations

import numpy as np

from . import widen64


def _window(windows, t, n):
    if windows is None:
        return 0, n
    lo, hi = int(windows[t][0]), int(windows[t][1])
    lo, hi = min(max(lo, 0), n), min(max(hi, 0), n)
    return lo, max(lo, hi)


def stca_attention(xt, X, Wq, Wk, Wv, cu_offsets, t_offsets, h, windows=None, scale=None):
    """Reordered single-query attention for every target.

    xt [T, D] target vectors; X [rows, D] history rows packed by
    ``cu_offsets`` [B+1]; ``t_offsets`` [B+1] groups the targets by user;
    Wq, Wk, Wv [D, D]; ``h`` heads; ``windows`` optional int [T, 2];
    ``scale`` defaults to 1/sqrt(D/h).  Returns out [T, D] float64."""
    xt, X, Wq, Wk, Wv = (widen64(a) for a in (xt, X, Wq, Wk, Wv))
    cu = np.asarray(cu_offsets, dtype=np.int64)
    tcu = np.asarray(t_offsets, dtype=np.int64)
    if windows is not None:
        windows = np.asarray(windows, dtype=np.int64)
    T, D = xt.shape
    dh = D // h
    c = 1.0 / np.sqrt(dh) if scale is None else float(scale)
    out = np.zeros((T, D))
    for b in range(len(cu) - 1):
        rows = X[cu[b]:cu[b + 1]]
        for t in range(int(tcu[b]), int(tcu[b + 1])):
            lo, hi = _window(windows, t, len(rows))
            Xw = rows[lo:hi]
            if len(Xw) == 0:
                continue
            q = xt[t] @ Wq
            for hh in range(h):
                cols = slice(hh * dh, (hh + 1) * dh)
                u = q[cols] @ Wk[:, cols].T
                s = c * (Xw @ u)
                a = np.exp(s - s.max())
                a /= a.sum()
                y = a @ Xw
                out[t, cols] = y @ Wv[:, cols]
    return out

