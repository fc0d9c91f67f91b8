"""GPU parity of the history-axis backward pass (sa_backward) against the
double-precision oracle (oracle/backward.py, pinned in tests/pins_backward.py).
The GPU recomputes the weights from the forward's lse and runs every product
on MFMA with bf16 operands (P, K, V, dS, the weights and score gradients),
so the bar is the bf16 one, per gradient: relative L2 <= 1e-2.  Masks and
layouts are checked bit-exactly (NaN-poisoned masked rows change nothing,
packed == dense, two runs are equal)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import backward as BW
import sketch_attention_flashsa_amd as sa
import workloads as W
from gpu_util import assert_parity, device, rel_l2

pytestmark = pytest.mark.gpu


def _upstream(w, seed):
    g = np.random.default_rng(seed)
    return torch.from_numpy(g.standard_normal((w["B"], w["H"], w["m"], w["dh"]), dtype=np.float32))


def run_bw(w, dS, P=None, K=None, V=None, mask="default", grad_dtype=None, raw=False):
    dev = device()
    P = (w["P"] if P is None else P).to(dev)
    K = (w["K"] if K is None else K).to(dev)
    V = (w["V"] if V is None else V).to(dev)
    mk = w.get("mask") if mask == "default" else mask
    mk = None if mk is None else mk.to(dev)
    kw = {"cu_offsets": w["cu_offsets"].to(dev)} if w["layout"] == "packed" else {"lengths": w["lengths"].to(dev)}
    S, lse = sa.sa_forward(P, K, V, mask=mk, return_lse=True, **kw)
    dP, dK, dV = sa.sa_backward(P, K, V, S, lse, dS.to(dev), mask=mk, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    if raw:
        return dP.cpu(), dK.cpu(), dV.cpu()
    return tuple(t.double().cpu().numpy() for t in (dP, dK, dV))


def oracle_bw(w, dS, P=None):
    P = w["P"] if P is None else P
    if w["layout"] == "packed":
        return BW.backward(P, w["K"], w["V"], dS, cu_offsets=w["cu_offsets"], mask=w.get("mask"))
    return BW.backward(P, w["K"], w["V"], dS, lengths=w["lengths"], mask=w.get("mask"))


def check(g, o, what):
    errs = []
    for a, b, n in zip(g, o, ("dP", "dK", "dV")):
        assert np.all(np.isfinite(a)), f"{what}: {n} not finite"
        errs.append(assert_parity(a, b, "bf16", f"{what} {n}"))
    print(f"{what}: relative L2 dP {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}", flush=True)


@pytest.mark.parametrize("dh,m,H", [(64, 128, 8), (32, 64, 4), (32, 256, 2), (64, 32, 3), (64, 256, 1), (32, 128, 5)])
def test_backward_shapes_ragged(dh, m, H):
    """Every compiled (dh, m), head counts that do and do not divide the dP
    kernel's heads per block, empty and single-row users, tails of the
    16- and 32-row tiles."""
    lengths = [700, 0, 1, 15, 17, 31, 33, 1200, 64]
    w = W.random_case(500 + dh + m + H, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16")
    dS = _upstream(w, 1)
    print(f"backward dh={dh} m={m} H={H} rows={sum(lengths)}", flush=True)
    check(run_bw(w, dS), oracle_bw(w, dS), f"dh={dh} m={m} H={H}")


@pytest.mark.parametrize("dh,m,H", [(64, 128, 8), (32, 256, 2), (32, 64, 3)])
def test_backward_bf16_gradients(dh, m, H):
    """dK and dV written as bf16: the fp32 gradients rounded to nearest even,
    bitwise (the same sums, only the store differs), and within the bf16 bar
    of the oracle; dP is unchanged."""
    lengths = [640, 0, 1, 17, 33, 1100]
    w = W.random_case(530 + dh + m, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16")
    dS = _upstream(w, 7)
    print(f"backward bf16 gradients dh={dh} m={m} H={H}", flush=True)
    f = run_bw(w, dS, raw=True)
    b = run_bw(w, dS, grad_dtype=torch.bfloat16, raw=True)
    assert b[1].dtype == torch.bfloat16 and b[2].dtype == torch.bfloat16
    assert torch.equal(f[0], b[0]), "dP must not depend on the gradient dtype"
    for n, x, y in (("dK", f[1], b[1]), ("dV", f[2], b[2])):
        assert torch.equal(x.to(torch.bfloat16).view(torch.int16), y.view(torch.int16)), f"{n}: not the RNE rounding"
    check(tuple(t.double().numpy() for t in b), oracle_bw(w, dS), f"bf16 gradients dh={dh} m={m} H={H}")


def test_backward_workload4_reduced():
    """The 100K workload's shape (H=8, m=128, dh=64) with two users capped at
    6000 rows."""
    w = W.make(4, B=2, max_len=6000)
    dS = _upstream(w, 2)
    check(run_bw(w, dS), oracle_bw(w, dS), "workload 4 reduced")


def test_backward_per_user_prototypes_and_scale():
    lengths = [400, 90, 1000]
    w = W.random_case(520, B=3, H=4, m=64, dh=32, lengths=lengths, dtype="bf16")
    g = np.random.default_rng(3)
    P = torch.from_numpy(g.standard_normal((3, 4, 64, 32), dtype=np.float32)).to(torch.bfloat16)
    dS = _upstream(w, 4)
    check(run_bw(w, dS, P=P), oracle_bw(w, dS, P=P), "per-user P")


def test_backward_mask_poison_dense_and_determinism():
    lengths = [300, 77, 900, 5]
    w = W.random_case(521, B=4, H=8, m=128, dh=64, lengths=lengths, dtype="bf16", mask_p=0.3)
    dS = _upstream(w, 5)
    g1 = run_bw(w, dS)
    check(g1, oracle_bw(w, dS), "masked")
    off = w["mask"].numpy() == 0
    assert np.all(g1[1][off] == 0) and np.all(g1[2][off] == 0), "masked rows must get zero dK, dV"
    K, V = w["K"].clone(), w["V"].clone()
    K[w["mask"] == 0] = float("nan")
    V[w["mask"] == 0] = float("nan")
    g2 = run_bw(w, dS, K=K, V=V)
    for a, b in zip(g1, g2):
        assert np.array_equal(np.nan_to_num(a, nan=7.0), np.nan_to_num(b, nan=7.0)) and np.all(np.isfinite(b))
    g3 = run_bw(w, dS)
    assert all(np.array_equal(a, b) for a, b in zip(g1, g3)), "two runs must be bitwise equal"
    # dense + lengths equals packed (dP bitwise, dK and dV on the valid rows)
    wp = W.random_case(522, B=3, H=4, m=64, dh=32, lengths=[500, 3, 260], dtype="bf16", layout="packed")
    wd = W.random_case(522, B=3, H=4, m=64, dh=32, lengths=[500, 3, 260], dtype="bf16", layout="dense")
    dS2 = _upstream(wp, 6)
    gp, gd = run_bw(wp, dS2), run_bw(wd, dS2)
    assert np.array_equal(gp[0], gd[0]), "dP: packed and dense must agree bitwise"
    cu = wp["cu_offsets"].tolist()
    for b, n in enumerate([500, 3, 260]):
        assert np.array_equal(gd[1][b, :n], gp[1][cu[b]:cu[b] + n])
        assert np.array_equal(gd[2][b, :n], gp[2][cu[b]:cu[b] + n])


@pytest.mark.slow
def test_backward_workload4_full_size_sampled():
    """The full 100K workload (16 users x 100,000 rows) in one call; the oracle
    recomputes three (user, head) pairs exactly (every row of the user)."""
    w = W.make(4, threads=16)
    dS = _upstream(w, 7)
    dP, dK, dV = run_bw(w, dS)
    cu = w["cu_offsets"].tolist()
    for b, h in ((0, 0), (7, 5), (15, 7)):
        rows = slice(cu[b], cu[b + 1])
        Kb = w["K"][rows, h:h + 1].contiguous()
        Vb = w["V"][rows, h:h + 1].contiguous()
        Pb = w["P"][h:h + 1].contiguous()
        o = BW.backward(Pb, Kb, Vb, dS[b:b + 1, h:h + 1].numpy(), cu_offsets=np.array([0, cu[b + 1] - cu[b]]))
        assert rel_l2(dK[rows, h], o[1][:, 0]) <= 1e-2 and rel_l2(dV[rows, h], o[2][:, 0]) <= 1e-2, (b, h)
