"""Pins for the backward oracle (``oracle/backward.py``): checks against
things other than that oracle.  Every pin takes the module to check (the real
one by default), so ``test_backward_oracle.py`` runs them on mutated copies.

  library_*   torch autograd in float64 through softmax and matmul (another
              implementation of the same derivative)
  fd_*        central finite differences of the forward oracle (the pinned C
              code) on tiny inputs
  inv_*       a common shift of a user's keys does not change S, so the
              user's dK sums to zero; the weights sum to one, so the user's dV
              sums to sum_j dS_j; masked rows and padding get zero gradients;
              linearity in dS; users do not interact
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import backward as BACKWARD
import workloads as W


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


def _case(seed, B=3, H=2, m=3, dh=4, lengths=(5, 1, 7), layout="packed", mask_p=0.0, per_user=False, std=1.0):
    w = W.random_case(seed, B=B, H=H, m=m, dh=dh, lengths=list(lengths), dtype="f32", layout=layout, mask_p=mask_p,
                      std=std)
    rng = np.random.default_rng(seed + 1000)
    w["dS"] = rng.standard_normal((B, H, m, dh))
    if per_user:
        w["P"] = torch.from_numpy(rng.standard_normal((B, H, m, dh)).astype(np.float32))
    return w


def _bw(R, w, **kw):
    if w["layout"] == "packed":
        return R.backward(w["P"], w["K"], w["V"], w["dS"], cu_offsets=w["cu_offsets"], mask=w.get("mask"), **kw)
    return R.backward(w["P"], w["K"], w["V"], w["dS"], lengths=w["lengths"], mask=w.get("mask"), **kw)


def _torch_grads(w, scale=None):
    """Autograd of sum(S * dS) through torch's softmax and matmul (float64)."""
    P = w["P"].double().clone().requires_grad_(True)
    K = w["K"].double().clone().requires_grad_(True)
    V = w["V"].double().clone().requires_grad_(True)
    cu = w["cu_offsets"].tolist()
    H, dh = K.shape[1], K.shape[2]
    c = scale if scale is not None else dh ** -0.5
    mask = w.get("mask")
    total = 0.0
    for b in range(len(cu) - 1):
        idx = torch.arange(cu[b], cu[b + 1])
        if mask is not None:
            idx = idx[mask[idx] != 0]
        if idx.numel() == 0:
            continue
        for h in range(H):
            Pj = P[h] if P.dim() == 3 else P[b, h]
            A = torch.softmax(c * Pj @ K[idx, h].T, dim=1)
            total = total + (A @ V[idx, h] * torch.from_numpy(w["dS"][b, h])).sum()
    total.backward()
    return P.grad.numpy(), K.grad.numpy(), V.grad.numpy()


# ---------------------------------------------------------------- library
def library_autograd_shared_p(R=BACKWARD):
    w = _case(1, B=3, H=2, m=4, dh=8, lengths=(9, 1, 14))
    got = _bw(R, w)
    ref = _torch_grads(w)
    for g, r, n in zip(got, ref, ("dP", "dK", "dV")):
        assert _rel(g, r) < 1e-12, (n, _rel(g, r))


def library_autograd_per_user_masked_scaled(R=BACKWARD):
    w = _case(2, B=3, H=3, m=5, dh=4, lengths=(11, 6, 3), mask_p=0.3, per_user=True, std=2.0)
    got = _bw(R, w, scale=0.37)
    ref = _torch_grads(w, scale=0.37)
    for g, r, n in zip(got, ref, ("dP", "dK", "dV")):
        assert _rel(g, r) < 1e-12, (n, _rel(g, r))


# ------------------------------------------------------- finite differences
def fd_against_forward_oracle(R=BACKWARD):
    w = _case(3, B=2, H=1, m=2, dh=3, lengths=(4, 3))
    dP, dK, dV = _bw(R, w)
    G = w["dS"]

    def loss(P, K, V):
        S, _ = oracle.forward(P, K, V, cu_offsets=w["cu_offsets"])
        return float((S * G).sum())

    P0, K0, V0 = (w[k].double().numpy() for k in ("P", "K", "V"))
    eps = 1e-6
    for name, X, grad in (("P", P0, dP), ("K", K0, dK), ("V", V0, dV)):
        num = np.zeros_like(X)
        it = np.nditer(X, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            Xp, Xm = X.copy(), X.copy()
            Xp[i] += eps
            Xm[i] -= eps
            args_p = {"P": P0, "K": K0, "V": V0}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            num[i] = (loss(**args_p) - loss(**args_m)) / (2 * eps)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), (name, np.abs(grad - num).max())


# ------------------------------------------------------------- invariants
def inv_key_shift_and_weight_sums(R=BACKWARD):
    w = _case(4, B=3, H=2, m=4, dh=6, lengths=(8, 5, 12))
    dP, dK, dV = _bw(R, w)
    cu = w["cu_offsets"].tolist()
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        assert np.allclose(dK[sl].sum(axis=0), 0.0, atol=1e-12), "a user's dK must sum to zero"
        assert np.allclose(dV[sl].sum(axis=0), w["dS"][b].sum(axis=1), atol=1e-12), "dV sums to sum_j dS_j"


def inv_mask_padding_and_isolation(R=BACKWARD):
    w = _case(5, B=3, H=2, m=3, dh=4, lengths=(7, 9, 4), mask_p=0.4)
    dP, dK, dV = _bw(R, w)
    off = w["mask"].numpy() == 0
    assert np.all(dK[off] == 0) and np.all(dV[off] == 0), "masked rows get zero gradients"
    # dense layout with padding: padded rows zero, valid rows equal to packed
    wd = _case(5, B=3, H=2, m=3, dh=4, lengths=(7, 9, 4), layout="dense")
    wp = _case(5, B=3, H=2, m=3, dh=4, lengths=(7, 9, 4))
    gd, gp = _bw(R, wd), _bw(R, wp)
    assert _rel(gd[0], gp[0]) < 1e-14
    for b, n in enumerate((7, 9, 4)):
        lo = sum((7, 9, 4)[:b])
        assert np.allclose(gd[1][b, :n], gp[1][lo:lo + n], rtol=1e-14, atol=0)
        assert np.all(gd[1][b, n:] == 0) and np.all(gd[2][b, n:] == 0)
    # changing user 1's keys leaves user 0's and 2's dK, dV unchanged
    w2 = dict(wp)
    K = wp["K"].clone()
    K[7:16] = -3 * K[7:16]
    w2["K"] = K
    g2 = _bw(R, w2)
    assert np.array_equal(g2[1][:7], gp[1][:7]) and np.array_equal(g2[2][16:], gp[2][16:])


def inv_linear_in_upstream(R=BACKWARD):
    w = _case(6, B=2, H=2, m=3, dh=4, lengths=(6, 5))
    g1 = _bw(R, w)
    w2 = dict(w, dS=w["dS"] * -2.5)
    g2 = _bw(R, w2)
    for a, b in zip(g1, g2):
        assert np.allclose(b, -2.5 * a, rtol=1e-13, atol=1e-15)


def inv_single_row_user(R=BACKWARD):
    # one valid row: A = 1 for every prototype, so dV = sum_j dS_j and every
    # score gradient vanishes (dK = 0, dP = 0)
    w = _case(7, B=1, H=2, m=4, dh=3, lengths=(1,))
    dP, dK, dV = _bw(R, w)
    assert np.allclose(dV[0], w["dS"][0].sum(axis=1), atol=1e-14)
    assert np.allclose(dK, 0, atol=1e-14) and np.allclose(dP, 0, atol=1e-14)


ALL_BACKWARD_PINS = [
    library_autograd_shared_p, library_autograd_per_user_masked_scaled, fd_against_forward_oracle,
    inv_key_shift_and_weight_sums, inv_mask_padding_and_isolation, inv_linear_in_upstream, inv_single_row_user,
]
