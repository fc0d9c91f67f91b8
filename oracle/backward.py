"""Double-precision oracle for the Sketch Attention backward pass, history
axis (test infrastructure only: ``tests/``, ``__graft_entry__.smoke()`` and the
CPU baseline of ``bench.py`` may use it; the GPU library never does).

The forward map is the one of section 3.1 of the SequenceO1 paper read along
the history axis (appendix A.4 writes it as a length-wise projection): per
user b, head h and prototype j,

    s_ji = c P_j . K_i          (c = 1/sqrt(dh) unless given)
    A_ji = exp(s_ji) / sum_i' exp(s_ji')     over the user's valid rows i
    S_j  = sum_i A_ji V_i

The paper trains SA end to end; its gradient, for an upstream gradient dS
(same shape as S), is the chain rule through the weighted sum and the
softmax, written out here with no reordering:

    dV_i  = sum_j A_ji dS_j
    dA_ji = dS_j . V_i
    ds_ji = A_ji (dA_ji - sum_i' A_ji' dA_ji')
    dK_i  = c sum_j ds_ji P_j
    dP_j  = c sum_i ds_ji K_i      (summed over users when P is shared)

Rows outside every user, masked rows and dense padding get dK = dV = 0.
Inputs stored in bf16 or fp32 are widened exactly; everything is float64.
"""
from __future__ import annotations

import numpy as np

from . import widen64


def _user_rows(b, cu, lengths, L_max, mask):
    if cu is not None:
        rows = np.arange(int(cu[b]), int(cu[b + 1]))
    else:
        n = L_max if lengths is None else max(0, min(int(lengths[b]), L_max))
        rows = b * L_max + np.arange(n)
    if mask is not None:
        rows = rows[np.asarray(mask).reshape(-1)[rows] != 0]
    return rows


def backward(P, K, V, dS, cu_offsets=None, lengths=None, mask=None, scale=None):
    """Gradients of S with respect to P, K and V.

    P [H, m, dh] (shared) or [B, H, m, dh] (per user); K, V packed
    [rows, H, dh] with ``cu_offsets`` [B+1], or dense [B, L_max, H, dh] with
    optional ``lengths``; ``mask`` per row (packed [rows], dense [B, L_max]);
    dS [B, H, m, dh].  Returns (dP shaped like P, dK and dV shaped like K),
    float64."""
    Pd, Kd, Vd, dSd = widen64(P), widen64(K), widen64(V), widen64(dS)
    dense = cu_offsets is None
    if dense:
        B, L_max, H, dh = Kd.shape
        Kf, Vf = Kd.reshape(B * L_max, H, dh), Vd.reshape(B * L_max, H, dh)
        cu = None
    else:
        H, dh = Kd.shape[1:]
        Kf, Vf = Kd, Vd
        cu = np.asarray(cu_offsets, dtype=np.int64)
        B, L_max = len(cu) - 1, 0
    m = Pd.shape[-2]
    c = 1.0 / np.sqrt(dh) if scale is None else float(scale)
    dP = np.zeros_like(Pd)
    dK = np.zeros_like(Kf)
    dV = np.zeros_like(Vf)
    for b in range(B):
        rows = _user_rows(b, cu, lengths, L_max, mask)
        if rows.size == 0:
            continue
        for h in range(H):
            Pj = Pd[h] if Pd.ndim == 3 else Pd[b, h]                 # [m, dh]
            Kb, Vb = Kf[rows, h], Vf[rows, h]                        # [n, dh]
            s = c * (Pj @ Kb.T)                                      # [m, n]
            s = s - s.max(axis=1, keepdims=True)
            A = np.exp(s)
            A /= A.sum(axis=1, keepdims=True)
            G = dSd[b, h]                                            # [m, dh]
            dV[rows, h] += A.T @ G
            dA = G @ Vb.T                                            # [m, n]
            ds = A * (dA - (A * dA).sum(axis=1, keepdims=True))
            dK[rows, h] += c * (ds.T @ Pj)
            if Pd.ndim == 3:
                dP[h] += c * (ds @ Kb)
            else:
                dP[b, h] += c * (ds @ Kb)
    if dense:
        dK, dV = dK.reshape(Kd.shape), dV.reshape(Vd.shape)
    return dP, dK, dV
