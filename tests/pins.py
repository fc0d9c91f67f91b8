"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin is a plain function that raises AssertionError when the oracle is
wrong.  ``test_oracle_pins.py`` runs them one by one; ``test_oracle_mutants.py``
plants mistakes in copies of the oracle's C source and checks that at least
one pin rejects every mutant.

What pins what (definitions: SequenceO1 paper, section 3.1 and appendix A.4):
  brute_*            50-digit mpmath implementation with materialised scores
  library_*          torch's scaled_dot_product_attention (float64, CPU) and
                     scipy.special.softmax / logsumexp: the history axis IS
                     single-query-block attention with queries P, so a library
                     routine computes it independently
  closed-form pins   P = 0 (mean), L = 1 (identity), L = 2 (logistic weights),
                     constant V
  invariants         shift of K (history) / of P (prototype), permutation of a
                     user's rows, linearity and convex hull in V, weights that
                     sum to one on the normalised axis, padding and masking,
                     cross-user isolation, large score offsets (no overflow)
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle import brute
import workloads as W


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b.ravel()), 1e-300)
    return np.linalg.norm((a - b).ravel()) / den


def _mp_to_np(x):
    if isinstance(x, list):
        return np.array([_mp_to_np(y) for y in x], dtype=np.float64)
    return float(x)


def _case(seed, B=3, H=2, m=3, dh=4, lengths=(5, 1, 9), dtype="f32", layout="packed", mask_p=0.0, std=1.0):
    return W.random_case(seed, B=B, H=H, m=m, dh=dh, lengths=list(lengths), dtype=dtype, layout=layout,
                         mask_p=mask_p, std=std)


# ------------------------------------------------------------- brute force
def _brute_compare(w, norm):
    P = w["P"].double().numpy()
    if w["layout"] == "packed":
        K = w["K"].double().numpy()
        V = w["V"].double().numpy()
        mask = None if "mask" not in w else w["mask"].numpy()
        S_b, A_b, L_b = brute.sketch_packed(P, K, V, w["cu_offsets"].numpy(), mask=mask, norm=norm)
        S_o, l_o = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=w.get("mask"), norm=norm)
    else:
        B, Lm = w["K"].shape[:2]
        K = w["K"].double().reshape(B * Lm, w["H"], w["dh"]).numpy()
        V = w["V"].double().reshape(B * Lm, w["H"], w["dh"]).numpy()
        mask = None if "mask" not in w else w["mask"].reshape(-1).numpy()
        S_b, A_b, L_b = brute.sketch_dense(P, K, V, B, Lm, lengths=w["lengths"].numpy(), mask=mask, norm=norm)
        S_o, l_o = oracle.forward(w["P"], w["K"], w["V"], lengths=w["lengths"], mask=w.get("mask"), norm=norm)
    S_b = _mp_to_np(S_b)
    assert _rel(S_o, S_b) <= 1e-12, f"oracle vs brute force: {_rel(S_o, S_b):.3e}"
    if norm == "history":
        Lb = _mp_to_np(L_b)
        fin = np.isfinite(Lb)
        assert np.array_equal(fin, np.isfinite(l_o)), "empty users must give lse = -inf"
        assert np.max(np.abs(l_o[fin] - Lb[fin]), initial=0.0) <= 1e-12, "lse vs brute force"


def brute_history_packed():
    for seed in (11, 12):
        _brute_compare(_case(seed), "history")


def brute_history_dense_lengths():
    _brute_compare(_case(13, layout="dense", lengths=(4, 0, 7)), "history")


def brute_history_masked():
    _brute_compare(_case(14, lengths=(8, 6, 10), mask_p=0.3), "history")


def brute_prototype_packed():
    _brute_compare(_case(15, lengths=(6, 3, 2)), "prototype")
    _brute_compare(_case(16, lengths=(5, 4, 3), mask_p=0.3, layout="dense"), "prototype")


def brute_bf16_inputs():
    _brute_compare(_case(17, dtype="bf16", lengths=(7, 2, 5)), "history")


def brute_per_user_prototypes():
    """P [B, H, m, dh] (one prototype set per user, as stacked refinement
    feeds them): the full forward and sampled rows against brute force."""
    w = _case(18, lengths=(6, 1, 9), mask_p=0.2)
    rng = np.random.default_rng(18)
    Pu = torch.from_numpy(rng.standard_normal((3, 2, 3, 4)).astype(np.float32))
    K, V, cu, mk = w["K"], w["V"], w["cu_offsets"], w["mask"]
    S_b, _, L_b = brute.sketch_packed(Pu.double().numpy(), K.double().numpy(), V.double().numpy(), cu.numpy(),
                                      mask=mk.numpy())
    S_b, L_b = _mp_to_np(S_b), _mp_to_np(L_b)
    S_o, l_o = oracle.forward(Pu, K, V, cu_offsets=cu, mask=mk)
    assert _rel(S_o, S_b) <= 1e-12, f"per-user P vs brute force: {_rel(S_o, S_b):.3e}"
    fin = np.isfinite(L_b)
    assert np.array_equal(fin, np.isfinite(l_o)) and np.max(np.abs(l_o[fin] - L_b[fin]), initial=0.0) <= 1e-12
    bhj = [(0, 1, 2), (2, 0, 1), (1, 1, 0)]
    o, ls = oracle.forward_sample(Pu, K, V, bhj, cu_offsets=cu, mask=mk)
    for t, (b, h, j) in enumerate(bhj):
        assert _rel(o[t], S_b[b, h, j]) <= 1e-12, "per-user P: sampled row vs brute force"


def brute_fused_values_are_x():
    """The fused entry with Wv = None (V = X: the paper's sketch aggregates X
    itself, section 3.1): full forward and sampled rows, with and without a
    mask, against brute force with every product an mpf."""
    rng = np.random.default_rng(6)
    bf = torch.bfloat16
    X = torch.from_numpy(rng.standard_normal((11, 8)).astype(np.float32)).to(bf)
    Wk = torch.from_numpy((rng.standard_normal((8, 8)) / 3).astype(np.float32)).to(bf)
    P = torch.from_numpy(rng.standard_normal((2, 3, 4)).astype(np.float32)).to(bf)
    cu = torch.tensor([0, 4, 4, 11], dtype=torch.int32)
    mk = torch.from_numpy((rng.uniform(size=11) > 0.3).astype(np.uint8))
    for mask in (None, mk):
        S_b, _, _ = brute.fused(X.double().numpy(), Wk.double().numpy(), None, P.double().numpy(), cu.numpy(),
                                mask=None if mask is None else mask.numpy())
        S_b = _mp_to_np(S_b)
        S_o, _ = oracle.fused_forward(X, Wk, None, P, cu, mask=mask)
        assert _rel(S_o, S_b) <= 1e-12, f"fused V = X vs brute force: {_rel(S_o, S_b):.3e}"
        bhj = [(0, 1, 2), (2, 0, 0), (2, 1, 1), (1, 0, 0)]
        o, _ = oracle.fused_forward_sample(X, Wk, None, P, cu, bhj, mask=mask)
        for t, (b, h, j) in enumerate(bhj):
            assert np.max(np.abs(o[t] - S_b[b, h, j])) <= 1e-12 * max(1.0, np.max(np.abs(S_b))), \
                "fused V = X: sampled row vs brute force"


# -------------------------------------------------------- library routines
def library_sdpa_history():
    """History axis == attention with the prototypes as queries (torch SDPA, float64)."""
    w = _case(21, B=3, H=3, m=7, dh=16, lengths=(50, 1, 33))
    S_o, l_o = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    cu = w["cu_offsets"].tolist()
    for b in range(3):
        for h in range(3):
            q = w["P"][h].double()[None, None]                      # [1,1,m,dh]
            k = w["K"][cu[b]:cu[b + 1], h].double()[None, None]      # [1,1,L,dh]
            v = w["V"][cu[b]:cu[b + 1], h].double()[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0].numpy()
            assert _rel(S_o[b, h], ref) <= 1e-12, f"SDPA mismatch b={b} h={h}"
            s = (w["P"][h].double() @ w["K"][cu[b]:cu[b + 1], h].double().T).numpy() / math.sqrt(16)
            from scipy.special import logsumexp
            assert np.max(np.abs(l_o[b, h] - logsumexp(s, axis=1))) <= 1e-12, "lse vs scipy logsumexp"


def library_scipy_both_axes():
    """Both axes against scipy.special.softmax on the materialised score matrix."""
    from scipy.special import softmax
    w = _case(22, B=2, H=2, m=5, dh=8, lengths=(12, 20), std=2.0)
    cu = w["cu_offsets"].tolist()
    for norm, axis in (("history", 1), ("prototype", 0)):
        S_o, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], norm=norm)
        for b in range(2):
            for h in range(2):
                Pm = w["P"][h].double().numpy()
                Km = w["K"][cu[b]:cu[b + 1], h].double().numpy()
                Vm = w["V"][cu[b]:cu[b + 1], h].double().numpy()
                A = softmax(Pm @ Km.T / math.sqrt(8), axis=axis)
                assert _rel(S_o[b, h], A @ Vm) <= 1e-12, f"{norm}: scipy mismatch"
                A_o = oracle.assignment(w["P"], w["K"], b, h, cu_offsets=w["cu_offsets"], norm=norm)
                assert np.max(np.abs(A_o - A)) <= 1e-13, f"{norm}: materialised A mismatch"


def library_projection():
    """Fused-projection oracle: K = X Wk, V = X Wv against numpy matmul."""
    rng = np.random.default_rng(5)
    X = torch.from_numpy(rng.standard_normal((17, 16)).astype(np.float32)).to(torch.bfloat16)
    Wk = torch.from_numpy((rng.standard_normal((16, 8)) / 4).astype(np.float32)).to(torch.bfloat16)
    Wv = torch.from_numpy((rng.standard_normal((16, 8)) / 4).astype(np.float32)).to(torch.bfloat16)
    P = torch.from_numpy(rng.standard_normal((2, 3, 4)).astype(np.float32)).to(torch.bfloat16)
    cu = torch.tensor([0, 9, 17], dtype=torch.int32)
    Kp = oracle.project(X, Wk)
    assert np.max(np.abs(Kp - X.double().numpy() @ Wk.double().numpy())) <= 1e-12, "projection vs numpy"
    S_f, _ = oracle.fused_forward(X, Wk, Wv, P, cu)
    Kd = torch.from_numpy(X.double().numpy() @ Wk.double().numpy()).reshape(17, 2, 4)
    Vd = torch.from_numpy(X.double().numpy() @ Wv.double().numpy()).reshape(17, 2, 4)
    S_r, _ = oracle.forward(P.double(), Kd, Vd, cu_offsets=cu)
    assert _rel(S_f, S_r) <= 1e-13, "fused forward vs projection + forward"
    o, _ = oracle.fused_forward_sample(X, Wk, Wv, P, cu, [(1, 1, 2), (0, 0, 0)])
    assert _rel(o[0], S_f[1, 1, 2]) <= 1e-13 and _rel(o[1], S_f[0, 0, 0]) <= 1e-13, "fused sample"


# ------------------------------------------------------------ closed forms
def closed_p_zero_is_mean():
    w = _case(31, lengths=(6, 1, 11), mask_p=0.25)
    w["P"] = torch.zeros_like(w["P"])
    cu = w["cu_offsets"].tolist()
    mk = w["mask"].numpy()
    S, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=w["mask"])
    Sp, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=w["mask"], norm="prototype")
    for b in range(3):
        rows = [r for r in range(cu[b], cu[b + 1]) if mk[r]]
        for h in range(2):
            if rows:
                mean = w["V"][rows, h].double().numpy().mean(axis=0)
                assert np.max(np.abs(S[b, h] - mean[None])) <= 1e-14, "P=0: history sketch must be the mean of V"
                total = w["V"][rows, h].double().numpy().sum(axis=0) / w["m"]
                assert np.max(np.abs(Sp[b, h] - total[None])) <= 1e-13, "P=0: prototype sketch must be sum(V)/m"
            else:
                assert np.all(S[b, h] == 0), "empty user must give S = 0"


def closed_single_row_is_identity():
    w = _case(32, lengths=(1, 1, 1), std=3.0)
    S, lse = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    for b in range(3):
        for h in range(2):
            assert np.array_equal(S[b, h], np.broadcast_to(w["V"][b, h].double().numpy(), S[b, h].shape)), \
                "L=1: sketch must equal the single value row exactly"
            s = (w["P"][h].double() @ w["K"][b, h].double()).numpy() / 2.0
            assert np.max(np.abs(lse[b, h] - s)) <= 1e-14, "L=1: lse must equal the score"


def closed_two_rows_logistic():
    w = _case(33, B=1, H=1, m=4, dh=4, lengths=(2,), std=1.5)
    S, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    P, K, V = (w[k].double().numpy() for k in ("P", "K", "V"))
    for j in range(4):
        s1, s2 = P[0, j] @ K[0, 0] / 2.0, P[0, j] @ K[1, 0] / 2.0
        sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
        expect = sig * V[0, 0] + (1 - sig) * V[1, 0]
        assert np.max(np.abs(S[0, 0, j] - expect)) <= 1e-14, "L=2: logistic closed form"


def closed_constant_v():
    w = _case(34, lengths=(9, 4, 6))
    c = torch.tensor([0.5, -1.25, 2.0, 3.0], dtype=torch.float32)
    w["V"][:] = c
    S, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    assert np.max(np.abs(S - c.double().numpy())) <= 1e-14, "history: constant V gives S = c"
    Sp, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], norm="prototype")
    cu = w["cu_offsets"].tolist()
    for b in range(3):
        for h in range(2):
            A = oracle.assignment(w["P"], w["K"], b, h, cu_offsets=w["cu_offsets"], norm="prototype")
            expect = A.sum(axis=1)[:, None] * c.double().numpy()[None]
            assert np.max(np.abs(Sp[b, h] - expect)) <= 1e-13, "prototype: S_j = c * sum_i A_ji"
            assert A.shape[1] == cu[b + 1] - cu[b]


# -------------------------------------------------------------- invariants
def inv_weights_sum_to_one():
    w = _case(41, lengths=(13, 2, 7), mask_p=0.2, std=2.0)
    for norm, axis in (("history", 1), ("prototype", 0)):
        for b in range(3):
            for h in range(2):
                A = oracle.assignment(w["P"], w["K"], b, h, cu_offsets=w["cu_offsets"], mask=w["mask"], norm=norm)
                if A.shape[1]:
                    assert np.max(np.abs(A.sum(axis=axis) - 1.0)) <= 1e-14, f"{norm}: weights must sum to one"
                    assert np.all(A >= 0)


def inv_shift():
    """History: K -> K + u (all rows of a user) leaves S unchanged, even when
    the shift makes the scores huge.  Prototype: P -> P + w (all prototypes)
    likewise.  Inputs are widened to double first so that the shift is exact."""
    w = _case(42, lengths=(10, 3, 8))
    P, K, V = w["P"].double(), w["K"].double(), w["V"].double()
    S0, _ = oracle.forward(P, K, V, cu_offsets=w["cu_offsets"])
    u = torch.full((2, 4), 200.0, dtype=torch.float64)
    S1, _ = oracle.forward(P, K + u[None], V, cu_offsets=w["cu_offsets"])
    assert _rel(S1, S0) <= 1e-9, "history axis must be invariant to a per-user shift of K"
    Sp0, _ = oracle.forward(P, K, V, cu_offsets=w["cu_offsets"], norm="prototype")
    Sp1, _ = oracle.forward(P + torch.full((2, 1, 4), 3.0, dtype=torch.float64), K, V,
                            cu_offsets=w["cu_offsets"], norm="prototype")
    assert _rel(Sp1, Sp0) <= 1e-11, "prototype axis must be invariant to a common shift of P"


def inv_large_scores_no_overflow():
    """Scores of order several hundred: exp would overflow without the max;
    checked against scipy's softmax on the materialised scores."""
    from scipy.special import softmax
    w = _case(43, lengths=(6, 5, 4), std=1.0)
    P = w["P"] * 300.0
    cu = w["cu_offsets"].tolist()
    for norm, axis in (("history", 1), ("prototype", 0)):
        S, _ = oracle.forward(P, w["K"], w["V"], cu_offsets=w["cu_offsets"], norm=norm)
        assert np.all(np.isfinite(S)), f"{norm}: large scores must not overflow"
        for b in range(3):
            for h in range(2):
                s = (P[h].double() @ w["K"][cu[b]:cu[b + 1], h].double().T).numpy() / 2.0
                ref = softmax(s, axis=axis) @ w["V"][cu[b]:cu[b + 1], h].double().numpy()
                assert _rel(S[b, h], ref) <= 1e-12, f"{norm}: large-score mismatch"


def inv_permutation():
    w = _case(44, lengths=(12, 5, 9), mask_p=0.2)
    S0, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=w["mask"])
    Sp0, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=w["mask"], norm="prototype")
    perm = []
    cu = w["cu_offsets"].tolist()
    rng = np.random.default_rng(0)
    for b in range(3):
        perm += list(cu[b] + rng.permutation(cu[b + 1] - cu[b]))
    perm = torch.tensor(perm)
    S1, _ = oracle.forward(w["P"], w["K"][perm], w["V"][perm], cu_offsets=w["cu_offsets"], mask=w["mask"][perm])
    Sp1, _ = oracle.forward(w["P"], w["K"][perm], w["V"][perm], cu_offsets=w["cu_offsets"], mask=w["mask"][perm],
                            norm="prototype")
    assert _rel(S1, S0) <= 1e-13 and _rel(Sp1, Sp0) <= 1e-13, "row order within a user must not matter"


def inv_linearity_and_hull():
    w = _case(45, lengths=(8, 3, 5))
    S1, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    V2 = torch.flip(w["V"], dims=[2]).contiguous()
    S2, _ = oracle.forward(w["P"], w["K"], V2, cu_offsets=w["cu_offsets"])
    S3, _ = oracle.forward(w["P"].double(), w["K"].double(), 2.0 * w["V"].double() - 0.5 * V2.double(),
                           cu_offsets=w["cu_offsets"])
    assert _rel(S3, 2.0 * S1 - 0.5 * S2) <= 1e-13, "sketch must be linear in V"
    cu = w["cu_offsets"].tolist()
    for b in range(3):
        Vb = w["V"][cu[b]:cu[b + 1]].double().numpy()
        lo, hi = Vb.min(axis=0), Vb.max(axis=0)          # [H, dh]
        assert np.all(S1[b] >= lo[:, None, :] - 1e-14) and np.all(S1[b] <= hi[:, None, :] + 1e-14), \
            "history sketch must lie in the convex hull of the user's values"


def inv_padding_and_masking():
    """dense + lengths + padding == packed; masked rows full of NaN change nothing
    and equal the compacted input."""
    w = _case(46, layout="dense", lengths=(7, 2, 5))
    B, Lm = w["K"].shape[:2]
    K, V = w["K"].clone(), w["V"].clone()
    for b, n in enumerate(w["lengths"].tolist()):
        K[b, n:] = float("nan")
        V[b, n:] = float("inf")
    Sd, _ = oracle.forward(w["P"], K, V, lengths=w["lengths"])
    rows = [b * Lm + i for b, n in enumerate(w["lengths"].tolist()) for i in range(n)]
    cu = torch.tensor([0] + list(np.cumsum(w["lengths"].numpy())), dtype=torch.int32)
    Sp, _ = oracle.forward(w["P"], K.reshape(B * Lm, 2, 4)[rows], V.reshape(B * Lm, 2, 4)[rows], cu_offsets=cu)
    assert np.array_equal(Sd, Sp), "dense+lengths must equal packed exactly"
    # masked rows poisoned with NaN == compacted copy
    w = _case(47, lengths=(9, 6, 4), mask_p=0.3)
    K, V = w["K"].clone(), w["V"].clone()
    mk = w["mask"].bool()
    K[~mk] = float("nan")
    V[~mk] = float("nan")
    Sm, _ = oracle.forward(w["P"], K, V, cu_offsets=w["cu_offsets"], mask=w["mask"])
    cu = w["cu_offsets"].tolist()
    keep = [r for r in range(cu[-1]) if mk[r]]
    new_cu = [0]
    for b in range(3):
        new_cu.append(new_cu[-1] + int(mk[cu[b]:cu[b + 1]].sum()))
    Sc, _ = oracle.forward(w["P"], w["K"][keep], w["V"][keep], cu_offsets=torch.tensor(new_cu, dtype=torch.int32))
    assert np.array_equal(Sm, Sc), "masked rows must be excluded exactly"
    ones = torch.ones_like(w["mask"])
    S1, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=ones)
    S0, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    assert np.array_equal(S1, S0), "an all-ones mask must equal no mask"


def inv_cross_user_isolation_and_empty():
    w = _case(48, lengths=(6, 0, 8))
    S0, l0 = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    assert np.all(S0[1] == 0) and np.all(np.isneginf(l0[1])), "empty user: S = 0, lse = -inf"
    cu = w["cu_offsets"].tolist()
    K2 = w["K"].clone()
    K2[cu[2]:cu[3]] = -K2[cu[2]:cu[3]] * 3
    S1, _ = oracle.forward(w["P"], K2, w["V"], cu_offsets=w["cu_offsets"])
    assert np.array_equal(S1[0], S0[0]) and not np.array_equal(S1[2], S0[2]), "users must not interact"


def inv_sample_equals_full():
    w = _case(49, B=3, H=2, m=5, dh=8, lengths=(40, 1, 17), dtype="bf16")
    S, l = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"])
    bhj = [(0, 1, 4), (1, 0, 0), (2, 1, 2)]
    o, ls = oracle.forward_sample(w["P"], w["K"], w["V"], bhj, cu_offsets=w["cu_offsets"])
    for t, (b, h, j) in enumerate(bhj):
        assert np.array_equal(o[t], S[b, h, j]) and ls[t] == l[b, h, j], "sampled rows must equal the full forward"


ALL_PINS = [
    brute_history_packed, brute_history_dense_lengths, brute_history_masked, brute_prototype_packed,
    brute_bf16_inputs, brute_per_user_prototypes, brute_fused_values_are_x, library_sdpa_history, library_scipy_both_axes, library_projection,
    closed_p_zero_is_mean, closed_single_row_is_identity, closed_two_rows_logistic, closed_constant_v,
    inv_weights_sum_to_one, inv_shift, inv_large_scores_no_overflow, inv_permutation,
    inv_linearity_and_hull, inv_padding_and_masking, inv_cross_user_isolation_and_empty,
    inv_sample_equals_full,
]
