"""GPU parity of STCA single-query attention (sa_stca_attention) against the
double-precision oracle (oracle/stca.py, pinned in tests/pins_stca.py).  The
GPU rounds q, u, the weights and alpha X to bf16 before their products (fp32
accumulation), so the bar is the bf16 one: relative L2 over the output
<= 1e-2, the oracle fed the same bf16 tensors."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import stca as ST
import sketch_attention_flashsa_amd as sa
import workloads as W
from gpu_util import assert_parity, device

pytestmark = pytest.mark.gpu


def run_stca(w, windows="default", t_offsets=None, xt=None, h=None, X=None):
    dev = device()
    win = w["windows"] if isinstance(windows, str) else windows
    out = sa.sa_stca_attention((w["xt"] if xt is None else xt).to(dev), w["X"].to(dev) if X is None else X,
                               w["Wq"].to(dev),
                               w["Wk"].to(dev), w["Wv"].to(dev), w["cu_offsets"].to(dev),
                               (w["t_offsets"] if t_offsets is None else t_offsets).to(dev), h or w["h"],
                               windows=None if win is None else win.to(dev))
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def oracle_stca(w, windows="default", t_offsets=None, xt=None, h=None):
    win = w["windows"] if isinstance(windows, str) else windows
    return ST.stca_attention(w["xt"] if xt is None else xt, w["X"], w["Wq"], w["Wk"], w["Wv"],
                             w["cu_offsets"].numpy(), (w["t_offsets"] if t_offsets is None else t_offsets).numpy(),
                             h or w["h"], windows=None if win is None else win.numpy())


@pytest.mark.parametrize("h", [16, 8])
def test_stca_ragged_users(h):
    """Users with no row, one row, rows around the 32-row tile, thousands of
    rows; target counts around the 16-target block (and a user with none)."""
    lengths = [0, 1, 31, 33, 700, 2048, 100]
    targets = [3, 5, 16, 17, 1, 40, 0]
    w = W.random_stca_case(900 + h, lengths=lengths, targets=targets, D=1024, h=h)
    print(f"stca h={h} rows={sum(lengths)} targets={sum(targets)}", flush=True)
    g = run_stca(w)
    o = oracle_stca(w)
    assert np.all(np.isfinite(g))
    assert np.all(g[:3] == 0), "a user with no rows gives 0"
    e = assert_parity(g, o, "bf16", f"stca h={h}")
    print(f"relative L2 {e:.2e}", flush=True)


@pytest.mark.parametrize("kind", ["random", "requests"])
def test_stca_windows(kind):
    """Request-aware windows: random [lo, hi) per target (empty ones included)
    and four nested requests per user."""
    lengths = [300, 1, 95, 1200]
    targets = [20, 2, 7, 33]
    w = W.random_stca_case(910, lengths=lengths, targets=targets, D=1024, h=16, windows=kind)
    g = run_stca(w)
    o = oracle_stca(w)
    empty = (w["windows"][:, 1] <= w["windows"][:, 0]).numpy()
    assert np.all(g[empty] == 0)
    assert_parity(g, o, "bf16", f"stca windows={kind}")


def test_stca_full_windows_equal_none_and_repeatable():
    """Windows that cover every user's rows change nothing, bitwise; two calls
    agree bitwise."""
    lengths = [77, 500]
    targets = [9, 18]
    w = W.random_stca_case(911, lengths=lengths, targets=targets, D=1024, h=16)
    full = torch.zeros((27, 2), dtype=torch.int32)
    full[:9, 1] = 77
    full[9:, 1] = 500
    a = run_stca(w)
    b = run_stca(w, windows=full)
    c = run_stca(w)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_stca_orphan_targets():
    """Targets before the first user's and after the last user's get 0."""
    lengths = [40, 60]
    w = W.random_stca_case(912, lengths=lengths, targets=[5, 4], D=1024, h=16)
    xt = torch.cat([w["xt"][:2], w["xt"], w["xt"][:3]])            # T = 14
    toff = torch.tensor([2, 7, 11], dtype=torch.int32)
    g = run_stca(w, xt=xt, t_offsets=toff)
    o = oracle_stca(w, xt=xt, t_offsets=toff)
    assert np.all(g[:2] == 0) and np.all(g[11:] == 0)
    assert_parity(g, o, "bf16", "stca orphan targets")


def test_stca_sketch_branch_workload_sampled():
    """The benchmarked sketch-branch shape (64 users x 1,024 sketch rows,
    40 targets each, D = 1024, h = 16) in the launch configuration the bench
    times; 3 users' outputs against the oracle (computed for those users
    only), and the rest finite."""
    B, L, R = 64, 1024, 40
    w = W.random_stca_case(913, lengths=[L] * B, targets=[R] * B, D=1024, h=16)
    g = run_stca(w)
    assert np.all(np.isfinite(g))
    for b in (0, 37, 63):
        sub = dict(w)
        sub["X"] = w["X"][b * L:(b + 1) * L]
        sub["cu_offsets"] = torch.tensor([0, L], dtype=torch.int32)
        sub["t_offsets"] = torch.tensor([0, R], dtype=torch.int32)
        o = oracle_stca(sub, xt=w["xt"][b * R:(b + 1) * R])
        assert_parity(g[b * R:(b + 1) * R], o, "bf16", f"stca sketch workload user {b}")


def test_stca_strided_rows_many_users_dh128():
    """History rows as a view of a wider buffer (x_row_stride > D), 1,100
    users (the block table's prefix runs over two 1,024-user passes), a
    user with no targets between users with targets, and h = 8 (dh = 128)
    with request windows."""
    rng = np.random.default_rng(914)
    B = 1100
    lengths = rng.integers(0, 40, size=B)
    targets = rng.integers(0, 3, size=B)
    targets[[5, 600, 1099]] = [17, 33, 1]
    w = W.random_stca_case(914, lengths=lengths.tolist(), targets=targets.tolist(), D=1024, h=8, windows="requests")
    dev = device()
    wide = torch.zeros((w["X"].shape[0], 1024 + 64), dtype=torch.bfloat16, device=dev)
    wide[:, :1024] = w["X"].to(dev)
    wide[:, 1024:] = float("nan")                        # never read
    g = run_stca(w, X=wide[:, :1024])
    o = oracle_stca(w)
    assert np.all(np.isfinite(g))
    assert_parity(g, o, "bf16", "stca strided rows, 1100 users, h=8")
