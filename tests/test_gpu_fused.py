"""GPU parity of the fused key/value projection entry (sa_forward_fused_proj)
against the double-precision oracle: K = X Wk and V = X Wv (or V = X) in
double with no rounding, then the history-axis forward.  The GPU rounds K, V
and the weights to bf16 before the MFMA products, so the bar is the bf16 one
(relative L2 over the output <= 1e-2, lse within 2e-2)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sketch_attention_flashsa_amd as sa
import workloads as W
from gpu_util import assert_lse, assert_parity, device

pytestmark = pytest.mark.gpu


def run_fused(w, use_wv=True, mask=None, P=None, **kw):
    dev = device()
    X, Wk, cu = w["X"].to(dev), w["Wk"].to(dev), w["cu_offsets"].to(dev)
    Pd = (w["P"] if P is None else P).to(dev)
    Wv = w["Wv"].to(dev) if use_wv else None
    mk = mask if mask is not None else w.get("mask")
    S, lse = sa.sa_forward_fused_proj(X, Wk, Wv, Pd, cu, mask=None if mk is None else mk.to(dev), return_lse=True,
                                      **kw)
    torch.cuda.synchronize()
    return S.double().cpu().numpy(), lse.double().cpu().numpy()


def oracle_fused(w, use_wv=True, mask=None):
    mk = mask if mask is not None else w.get("mask")
    return oracle.fused_forward(w["X"], w["Wk"], w["Wv"] if use_wv else None, w["P"], w["cu_offsets"], mask=mk)


def test_fused_workload5_reduced():
    """First 6 users of the fused workload, lengths capped at 2500 (several
    row ranges per user, ragged tails), W_V given."""
    w = W.make(5, B=6, max_len=2500)
    print(f"fused workload reduced: rows={int(w['lengths'].sum())}", flush=True)
    S, lse = run_fused(w)
    So, lo = oracle_fused(w)
    assert np.all(np.isfinite(S))
    assert_parity(S, So, "bf16", "fused workload, reduced")
    assert_lse(lse, lo, "bf16", "fused workload, reduced")


def test_fused_v_equals_x():
    """W_V omitted: the sketch aggregates X itself (needs H*dh == d_model)."""
    w = W.make(5, B=4, max_len=1500)
    S, lse = run_fused(w, use_wv=False)
    So, lo = oracle_fused(w, use_wv=False)
    assert_parity(S, So, "bf16", "fused, V = X")
    assert_lse(lse, lo, "bf16", "fused, V = X")


@pytest.mark.parametrize("offset,ramp", [(100.0, 0.0), (-200.0, 0.0), (0.0, 0.05), (0.0, -0.05), (60.0, 0.02)])
def test_fused_running_maximum_moves(offset, ramp):
    """Scores far from 0, and scores that rise or fall along each user's rows.
    The fused kernel keeps each running maximum at 0 while the weights 2^s stay
    in range and moves it only where they would not, so these cases take the
    moves up (offset +100, rising ramps), the move down before any mass is
    summed (offset -200) and the lazy steps between.  Model channel 0 of X
    carries the shift: column h dh of W_K reads that channel alone (weight 1),
    channel 0 of every prototype is 4, so a row's base-2 scores move by
    offset + ramp * (its index in the user).  The scale is the float nearest
    1 / log2(e), for which the kernel's pre-scaled prototypes are exact, so
    scores of several hundred keep the lse bar."""
    d_model, H, m, dh = 128, 4, 64, 32
    unit_scale = float(np.float32(1.0) / np.float32(np.log2(np.e)))
    w = W.random_fused_case(211 + int(offset) + int(100 * ramp), B=3, H=H, m=m, dh=dh, d_model=d_model,
                            lengths=[3000, 777, 65])
    X, Wk, P = w["X"].float(), w["Wk"].float(), w["P"].float()
    cu = w["cu_offsets"].tolist()
    unit = 0.25                                       # X[:, 0] per base-2 unit of score
    for b in range(3):
        r = torch.arange(cu[b + 1] - cu[b], dtype=torch.float32)
        X[cu[b]:cu[b + 1], 0] = (offset + ramp * r) * unit
    Wk[0, :] = 0.0
    for h in range(H):
        Wk[:, h * dh] = 0.0
        Wk[0, h * dh] = 1.0
    # the other channels at the usual size of base-2 scores (the unit scale
    # drops the 1 / sqrt(dh)), so the rounding of the projected keys stays as
    # small against the lse bar as at the default scale
    P[:, :, 1:] *= 1.0 / np.sqrt(dh)
    P[:, :, 0] = 4.0
    w = dict(w, X=X.to(torch.bfloat16), Wk=Wk.to(torch.bfloat16), P=P.to(torch.bfloat16))
    S, lse = run_fused(w, scale=unit_scale)
    So, lo = oracle.fused_forward(w["X"], w["Wk"], w["Wv"], w["P"], w["cu_offsets"], scale=unit_scale)
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(lse))
    assert_parity(S, So, "bf16", f"fused, offset {offset}, ramp {ramp}")
    assert_lse(lse, lo, "bf16", f"fused, offset {offset}, ramp {ramp}")


@pytest.mark.parametrize("d_model,H,m", [(256, 8, 256), (256, 8, 128), (256, 8, 64), (128, 4, 256), (128, 4, 64),
                                         (256, 5, 128)])
def test_fused_shapes_ragged(d_model, H, m):
    """Every compiled (d_model, m) family, a head count that leaves idle waves
    (H = 5), empty users, single rows and lengths around the 32-row tile."""
    lengths = [1, 0, 31, 32, 33, 95, 700, 0, 64, 1311]
    w = W.random_fused_case(300 + m + H, B=len(lengths), H=H, m=m, dh=32, d_model=d_model, lengths=lengths)
    S, lse = run_fused(w)
    So, lo = oracle_fused(w)
    assert_parity(S, So, "bf16", f"fused d_model={d_model} H={H} m={m}")
    assert_lse(lse, lo, "bf16", f"fused d_model={d_model} H={H} m={m}")
    # empty users: S = 0 and lse = -inf exactly
    for b in (1, 7):
        assert np.all(S[b] == 0) and np.all(np.isneginf(lse[b]))
    # a single row: the sketch is that row's value (bf16-rounded V)
    V1 = oracle.project(w["X"][:1], w["Wv"]).reshape(H, 32)
    assert np.allclose(S[0], np.broadcast_to(V1[:, None, :], S[0].shape), rtol=1e-2, atol=1e-2)


def test_fused_small_chunks_match_default_split():
    """chunk_rows = 64 cuts every user into many segments; the merge must
    give the same sketch (to tolerance) as the default split."""
    w = W.random_fused_case(311, B=3, H=8, m=256, dh=32, d_model=256, lengths=[900, 5, 2000])
    S1, l1 = run_fused(w)
    S2, l2 = run_fused(w, chunk_rows=64)
    So, lo = oracle_fused(w)
    assert_parity(S2, So, "bf16", "fused, chunk_rows=64")
    assert_lse(l2, lo, "bf16", "fused, chunk_rows=64")
    assert_parity(S1, So, "bf16", "fused, default split")


@pytest.mark.parametrize("H,m,d_model", [(8, 256, 256), (8, 128, 256), (4, 256, 128)])
def test_fused_mask_poison_is_bit_exact(H, m, d_model):
    """Masked rows are never read as numbers: NaN in X at masked rows leaves
    the output bitwise unchanged; the result matches the oracle's mask.  The
    shapes cover both ways a tile's mask reaches the kernel (with the tile
    through LDS, and read directly where the LDS is full)."""
    w = W.random_fused_case(312 + m + d_model, B=4, H=H, m=m, dh=32, d_model=d_model,
                            lengths=[400, 77, 1000, 33], mask_p=0.3)
    S, lse = run_fused(w)
    X2 = w["X"].clone()
    X2[w["mask"] == 0] = float("nan")
    S2, lse2 = run_fused(dict(w, X=X2))
    assert np.array_equal(S, S2) and np.array_equal(lse, lse2), "masked NaN rows leaked"
    So, lo = oracle_fused(w)
    assert_parity(S, So, "bf16", "fused, masked")
    assert_lse(lse, lo, "bf16", "fused, masked")
    # an all-ones mask is the same as no mask, bitwise
    ones = torch.ones_like(w["mask"])
    Sa, la = run_fused(w, mask=ones)
    Sn, ln = run_fused(dict(w, mask=None))
    assert np.array_equal(Sa, Sn) and np.array_equal(la, ln)


def test_fused_rows_outside_users_are_ignored():
    """Rows before cu[0] and after cu[B] (NaN) are never read."""
    w = W.random_fused_case(313, B=3, H=8, m=128, dh=32, d_model=256, lengths=[300, 0, 450])
    S, lse = run_fused(w)
    pad = 37
    X = torch.full((w["X"].shape[0] + 2 * pad, 256), float("nan"), dtype=torch.bfloat16)
    X[pad:pad + w["X"].shape[0]] = w["X"]
    S2, lse2 = run_fused(dict(w, X=X, cu_offsets=w["cu_offsets"] + pad))
    assert np.array_equal(S, S2) and np.array_equal(lse, lse2)


def test_fused_determinism_and_isolation():
    w = W.random_fused_case(314, B=3, H=8, m=256, dh=32, d_model=256, lengths=[1200, 64, 800])
    S1, l1 = run_fused(w)
    S2, l2 = run_fused(w)
    assert np.array_equal(S1, S2) and np.array_equal(l1, l2), "two runs differ"
    # changing user 1's rows leaves users 0 and 2 bitwise unchanged
    X = w["X"].clone()
    c = w["cu_offsets"]
    X[c[1]:c[2]] = -X[c[1]:c[2]] * 3
    S3, _ = run_fused(dict(w, X=X))
    assert np.array_equal(S1[0], S3[0]) and np.array_equal(S1[2], S3[2])


def test_fused_per_user_prototypes():
    """P [B, H, m, dh]: each user equals a shared-P call with its prototypes."""
    w = W.random_fused_case(315, B=3, H=8, m=128, dh=32, d_model=256, lengths=[500, 1, 260], per_user_p=True)
    S, _ = run_fused(w)
    for b in range(3):
        Sb, _ = run_fused(w, P=w["P"][b])
        assert np.array_equal(S[b], Sb[b]), "per-user prototypes must match the shared call"


@pytest.mark.parametrize("H,dh,d_model,m", [(1, 128, 128, 1024), (2, 128, 256, 256)])
def test_fused_two_pass_production_shape(H, dh, d_model, m):
    """The paper's production shape (one head of width 128, 1024 prototypes,
    values = X, appendix G.5), where W_K is folded into the prototypes and K
    is never formed, and a two-head variant, where K = X Wk is projected into
    the workspace and the streaming forward runs on it."""
    lengths = [1200, 0, 1, 31, 33, 700, 64]
    w = W.random_fused_case(316 + m, B=len(lengths), H=H, m=m, dh=dh, d_model=d_model, lengths=lengths,
                            w_var=1.0 / d_model, mask_p=0.15)
    S, lse = run_fused(w, use_wv=False)
    So, lo = oracle_fused(w, use_wv=False)
    assert np.all(np.isfinite(S))
    assert_parity(S, So, "bf16", f"two-pass H={H} dh={dh} m={m}")
    assert_lse(lse, lo, "bf16", f"two-pass H={H} dh={dh} m={m}")
    # masked rows poisoned with NaN change nothing
    X2 = w["X"].clone()
    X2[w["mask"] == 0] = float("nan")
    S2, lse2 = run_fused(dict(w, X=X2), use_wv=False)
    assert np.array_equal(S, S2) and np.array_equal(lse, lse2), "masked NaN rows leaked"


def test_production_shape_full_size_sampled():
    """The production shape at the benchmark's size and launch configuration
    (16 users x 100,000 rows, one head of width 128, 1024 prototypes, V = X,
    keys X W_K folded into the prototypes): sampled (user, prototype) rows of
    the longest users against the oracle, which projects K itself."""
    B, L, m, dm = 16, 100_000, 1024, 128
    w = W.random_fused_case(8, B=1, H=1, m=m, dh=dm, d_model=dm, lengths=[1], w_var=1.0 / dm)
    g = torch.Generator().manual_seed(8)
    X = torch.randn(B * L, dm, generator=g).to(torch.bfloat16)
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32)
    full = dict(w, X=X, cu_offsets=cu, B=B, lengths=torch.full((B,), L, dtype=torch.int64))
    S, lse = run_fused(full, use_wv=False)
    assert np.all(np.isfinite(S))
    rng = np.random.default_rng(88)
    bhj = [(b, 0, int(rng.integers(m))) for b in (0, 7, 15) for _ in range(4)]
    o, lo = oracle.fused_forward_sample(X, w["Wk"], None, w["P"], cu, bhj)
    gsel = np.stack([S[b, h, j] for b, h, j in bhj])
    gl = np.array([lse[b, h, j] for b, h, j in bhj])
    assert_parity(gsel, o, "bf16", "production shape, sampled rows")
    assert_lse(gl, lo, "bf16", "production shape, sampled lse")


@pytest.mark.slow
def test_fused_workload5_full_size_sampled():
    """The full fused workload (128 users, 4.24M rows, X 2.17 GB) in the launch
    configuration the benchmark times; the oracle computes 24 sampled
    (user, head, prototype) rows one by one."""
    w = W.make(5, threads=16)
    S, lse = run_fused(w)
    assert np.all(np.isfinite(S))
    rng = np.random.default_rng(5)
    lens = w["lengths"].numpy()
    order = np.argsort(lens)
    users = list(order[:4]) + list(order[-4:]) + list(rng.choice(w["B"], 16, replace=False))
    bhj = [(int(b), int(rng.integers(w["H"])), int(rng.integers(w["m"]))) for b in users]
    o, lo = oracle.fused_forward_sample(w["X"], w["Wk"], w["Wv"], w["P"], w["cu_offsets"], bhj)
    g = np.stack([S[b, h, j] for b, h, j in bhj])
    gl = np.array([lse[b, h, j] for b, h, j in bhj])
    assert_parity(g, o, "bf16", "fused full size, sampled rows")
    assert_lse(gl, lo, "bf16", "fused full size, sampled lse")
