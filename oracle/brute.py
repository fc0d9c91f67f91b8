"""Brute-force Sketch Attention at 50 significant digits (test infrastructure only).

An independent second implementation used to pin the C oracle on tiny inputs.
It materialises every score and every assignment weight as an ``mpmath``
number with pure-Python loops, following the definitions of the SequenceO1
paper, section 3.1 (scores P W_Q (X W_K)^T / sqrt(d), prototype-normalised
assignment, sketch A X) and appendix A.4, with the history-axis reading as the
default.  It never calls the C oracle and shares no code with it.
"""
from __future__ import annotations

import mpmath

mpmath.mp.dps = 50


def _mp(x):
    """An mpf for a stored float (exact) or an mpf computed here (kept as is)."""
    return x if isinstance(x, mpmath.mpf) else mpmath.mpf(float(x))


def _user_rows(b, cu, lengths, L_max, mask):
    if cu is not None:
        rows = list(range(int(cu[b]), int(cu[b + 1])))
    else:
        n = L_max if lengths is None else max(0, min(int(lengths[b]), L_max))
        rows = [b * L_max + i for i in range(n)]
    if mask is not None:
        rows = [r for r in rows if int(mask[r]) != 0]
    return rows


def sketch_packed(P, K, V, cu, mask=None, norm="history", scale=None):
    """Packed layout: K, V [rows][H][dh]; cu [B+1].  See :func:`_sketch`."""
    return _sketch(P, K, V, len(cu) - 1, lambda b: _user_rows(b, cu, None, 0, mask), norm, scale)


def sketch_dense(P, K, V, B, L_max, lengths=None, mask=None, norm="history", scale=None):
    """Dense layout flattened to rows: K, V [B*L_max][H][dh]."""
    return _sketch(P, K, V, B, lambda b: _user_rows(b, None, lengths, L_max, mask), norm, scale)


def _sketch(P, K, V, B, rows_of, norm, scale):
    """P [H][m][dh], or [B][H][m][dh] with one prototype set per user (a
    numpy array of 4 dimensions); K, V [rows][H][dh] (any nested indexable of
    floats).

    Returns (S [B][H][m][dh], A, lse) as mpf: A[b][h] is the materialised
    [m][n_valid] assignment matrix; lse[b][h] is per prototype (history axis)
    or per valid token (prototype axis), natural log, scale included.
    """
    per_user = getattr(P, "ndim", 3) == 4
    P0 = P[0] if per_user else P
    H, m, dh = len(P0), len(P0[0]), len(P0[0][0])
    sc = mpmath.mpf(1) / mpmath.sqrt(dh) if scale is None else mpmath.mpf(scale)
    S, W, LSE = [], [], []
    P_all = P
    for b in range(B):
        P = P_all[b] if per_user else P_all
        rows = rows_of(b)
        Sb, Wb, Lb = [], [], []
        for h in range(H):
            # scores s[j][t] = scale * <P[h][j], K[row_t][h]>
            s = [[sc * mpmath.fsum(_mp(P[h][j][e]) * _mp(K[r][h][e])
                                   for e in range(dh)) for r in rows] for j in range(m)]
            n = len(rows)
            if norm == "history":
                A, lse = [], []
                for j in range(m):
                    if n == 0:
                        A.append([])
                        lse.append(mpmath.mpf("-inf"))
                        continue
                    e_ = [mpmath.exp(x) for x in s[j]]
                    Z = mpmath.fsum(e_)
                    A.append([x / Z for x in e_])
                    lse.append(mpmath.log(Z))
            else:
                A = [[mpmath.mpf(0)] * n for _ in range(m)]
                lse = []
                for t in range(n):
                    e_ = [mpmath.exp(s[j][t]) for j in range(m)]
                    Z = mpmath.fsum(e_)
                    for j in range(m):
                        A[j][t] = e_[j] / Z
                    lse.append(mpmath.log(Z))
            Sbh = [[mpmath.fsum(A[j][t] * _mp(V[rows[t]][h][e]) for t in range(n))
                    for e in range(dh)] for j in range(m)]
            Sb.append(Sbh)
            Wb.append(A)
            Lb.append(lse)
        S.append(Sb)
        W.append(Wb)
        LSE.append(Lb)
    return S, W, LSE


# ------------------------------------------- fused projection (tiny)
def fused(X, Wk, Wv, P, cu, mask=None, scale=None):
    """Keys K = X Wk and values V = X Wv -- or V = X itself when ``Wv`` is
    None, the paper's sketch of X (section 3.1) -- every product an mpf, then
    the history-axis sketch of :func:`sketch_packed`.  X [rows][d_model],
    Wk (and Wv) [d_model][H dh], P [H][m][dh]; head h is columns
    [h dh, (h+1) dh) of K and V (of X when V = X).  Returns (S, A, lse)."""
    H, dh = len(P), len(P[0][0])
    Xm = _mat(X)
    Km = _matmul(Xm, _mat(Wk))
    Vm = _matmul(Xm, _mat(Wv)) if Wv is not None else Xm
    K3 = [[[Km[r][h * dh + e] for e in range(dh)] for h in range(H)] for r in range(len(Xm))]
    V3 = [[[Vm[r][h * dh + e] for e in range(dh)] for h in range(H)] for r in range(len(Xm))]
    return sketch_packed(P, K3, V3, cu, mask=mask, scale=scale)


# ------------------------------------------------- stacked refinement (tiny)
def _mat(A):
    return [[mpmath.mpf(float(v)) for v in row] for row in A]


def _matmul(A, B):
    n, k, m = len(A), len(B), len(B[0])
    return [[mpmath.fsum(A[i][t] * B[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def _layer_norm_row(x, g, bta, eps):
    n = len(x)
    mu = mpmath.fsum(x) / n
    var = mpmath.fsum((v - mu) ** 2 for v in x) / n
    inv = 1 / mpmath.sqrt(var + eps)
    return [(x[i] - mu) * inv * g[i] + bta[i] for i in range(n)]


def refine(X, P0, layers, cu, H, eps=1e-5):
    """Section 3.3 of the SequenceO1 paper, one user at a time, every score
    and weight an mpf: Q = Xt Wq, K = X Wk, per head h (channels
    [h dh, (h+1) dh)) weights softmax over the user's rows of
    Q_h K_h^T / sqrt(dh), Xhat_h = weights X_h, then
    Xbar = LN(Xt + Xhat), Xt' = LN(Xbar + (silu(Xbar W1) * Xbar W3) W2).
    X [rows][d], P0 [k][d]; ``layers`` as in ``oracle.refine.refine`` (nested
    lists or arrays of floats).  Returns [B][k][d] mpf."""
    B = len(cu) - 1
    d = len(P0[0])
    dh = d // H
    sc = 1 / mpmath.sqrt(dh)
    out = []
    for b in range(B):
        rows = [_mat([X[r]])[0] for r in range(int(cu[b]), int(cu[b + 1]))]
        Xt = _mat(P0)
        for L in layers:
            Wq, Wk = _mat(L["Wq"]), _mat(L["Wk"])
            Q = _matmul(Xt, Wq)
            K = _matmul(rows, Wk) if rows else []
            k = len(Q)
            Xhat = [[mpmath.mpf(0)] * d for _ in range(k)]
            for h in range(H):
                c = range(h * dh, (h + 1) * dh)
                for j in range(k):
                    if not rows:
                        continue
                    s = [mpmath.fsum(Q[j][e] * K[i][e] for e in c) * sc for i in range(len(rows))]
                    M = max(s)
                    w = [mpmath.exp(v - M) for v in s]
                    Z = mpmath.fsum(w)
                    for e in c:
                        Xhat[j][e] = mpmath.fsum(w[i] * rows[i][e] for i in range(len(rows))) / Z
            g1, b1 = [mpmath.mpf(float(v)) for v in L["ln1_g"]], [mpmath.mpf(float(v)) for v in L["ln1_b"]]
            g2, b2 = [mpmath.mpf(float(v)) for v in L["ln2_g"]], [mpmath.mpf(float(v)) for v in L["ln2_b"]]
            Xbar = [_layer_norm_row([Xt[j][e] + Xhat[j][e] for e in range(d)], g1, b1, eps) for j in range(k)]
            A1 = _matmul(Xbar, _mat(L["W1"]))
            A3 = _matmul(Xbar, _mat(L["W3"]))
            Hid = [[A1[j][t] / (1 + mpmath.exp(-A1[j][t])) * A3[j][t] for t in range(len(A1[0]))] for j in range(k)]
            F = _matmul(Hid, _mat(L["W2"]))
            Xt = [_layer_norm_row([Xbar[j][e] + F[j][e] for e in range(d)], g2, b2, eps) for j in range(k)]
        out.append(Xt)
    return out


# ------------------------------------ STCA single-query attention (tiny)
def stca(xt, X, Wq, Wk, Wv, cu, tcu, h, windows=None):
    """Section 2.3 of the SequenceO1 paper written as it stands (no
    reordering), every number an mpf: per target q and head hh (channels
    c = [hh dh, (hh+1) dh)), keys K = X W_K[:, c] and values V = X W_V[:, c]
    of the rows in the target's window, weights softmax(q W_Q[:, c] K^T /
    sqrt(dh)), output weights V.  Returns [T][D] mpf (0 for targets with no
    row)."""
    T, D = len(xt), len(xt[0])
    dh = D // h
    sc = 1 / mpmath.sqrt(dh)
    out = [[mpmath.mpf(0)] * D for _ in range(T)]
    Wq_, Wk_, Wv_ = _mat(Wq), _mat(Wk), _mat(Wv)
    for b in range(len(cu) - 1):
        rows = [_mat([X[r]])[0] for r in range(int(cu[b]), int(cu[b + 1]))]
        for t in range(int(tcu[b]), int(tcu[b + 1])):
            lo, hi = 0, len(rows)
            if windows is not None:
                lo = min(max(int(windows[t][0]), 0), len(rows))
                hi = max(lo, min(max(int(windows[t][1]), 0), len(rows)))
            Xw = rows[lo:hi]
            if not Xw:
                continue
            q = _matmul(_mat([xt[t]]), Wq_)[0]
            for hh in range(h):
                c = range(hh * dh, (hh + 1) * dh)
                qh = [q[e] for e in c]
                K = [[mpmath.fsum(x[d] * Wk_[d][e] for d in range(D)) for e in c] for x in Xw]
                V = [[mpmath.fsum(x[d] * Wv_[d][e] for d in range(D)) for e in c] for x in Xw]
                s = [mpmath.fsum(qh[e] * k[e] for e in range(dh)) * sc for k in K]
                M = max(s)
                w = [mpmath.exp(v - M) for v in s]
                Z = mpmath.fsum(w)
                for i, e in enumerate(c):
                    out[t][e] = mpmath.fsum(w[r] * V[r][i] for r in range(len(Xw))) / Z
    return out
