"""GPU parity of stacked Sketch Attention refinement (sa_refine_forward)
against the double-precision oracle (oracle/refine.py, pinned in
tests/pins_refine.py).  The GPU rounds queries, keys, attention weights and
the FFN's inputs and hidden units to bf16 before each product (fp32
accumulation, fp32 layer norms), so the bar is the bf16 one: relative L2 over
the final sketch <= 1e-2."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import refine as R
import sketch_attention_flashsa_amd as sa
import workloads as W
from gpu_util import assert_parity, device

pytestmark = pytest.mark.gpu


def run_refine(w, eps=1e-5, layers=None, X=None, cu=None, mask="default"):
    dev = device()
    Ls = [{k: v.to(dev) for k, v in L.items()} for L in (layers or w["layers"])]
    mk = w.get("mask") if mask == "default" else mask
    out = sa.sa_refine_forward((w["X"] if X is None else X).to(dev), w["P0"].to(dev), Ls,
                               (w["cu_offsets"] if cu is None else cu).to(dev), w["H"],
                               mask=None if mk is None else mk.to(dev), eps=eps)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def oracle_refine(w, eps=1e-5, layers=None):
    return R.refine(w["X"], w["P0"], layers or w["layers"], w["cu_offsets"].numpy(), w["H"], mask=w.get("mask"),
                    eps=eps)


@pytest.mark.parametrize("d,H,m", [(256, 8, 256), (256, 8, 128), (128, 4, 64), (128, 4, 256)])
def test_refine_two_layers(d, H, m):
    """Two layers (the paper's N_sa = 2) on ragged users: empty, single-row,
    around the 32-row tile, and a few thousand rows."""
    lengths = [1500, 0, 1, 31, 33, 700, 2048]
    w = W.random_refine_case(400 + d + m, B=len(lengths), H=H, m=m, dh=d // H, lengths=lengths, n_layers=2)
    print(f"refine d={d} H={H} m={m} rows={sum(lengths)}", flush=True)
    g = run_refine(w)
    o = oracle_refine(w)
    assert np.all(np.isfinite(g))
    e = assert_parity(g, o, "bf16", f"refine d={d} H={H} m={m}")
    print(f"relative L2 {e:.2e}", flush=True)


def test_refine_one_and_three_layers_masked():
    lengths = [900, 5, 1200]
    w = W.random_refine_case(411, B=3, H=8, m=128, dh=32, lengths=lengths, n_layers=3, mask_p=0.25)
    for n in (1, 3):
        g = run_refine(w, layers=w["layers"][:n])
        o = oracle_refine(w, layers=w["layers"][:n])
        assert_parity(g, o, "bf16", f"refine {n} layer(s), masked")


def test_refine_fused_workload_reduced():
    """The fused workload's users (first 4, lengths capped at 3000) with two
    seeded layers."""
    w5 = W.make(5, B=4, max_len=3000)
    w = dict(w5, H=8, P0=W.random_refine_case(412, B=1, H=8, m=256, dh=32, lengths=[1])["P0"],
             layers=W.refine_layers(412, 256, 2))
    g = run_refine(w)
    o = oracle_refine(w)
    e = assert_parity(g, o, "bf16", "refine on the fused workload, reduced")
    print(f"relative L2 {e:.2e}", flush=True)


def test_refine_deterministic_isolated_and_poison():
    lengths = [600, 300, 800]
    w = W.random_refine_case(413, B=3, H=8, m=128, dh=32, lengths=lengths, n_layers=2, mask_p=0.2)
    g1 = run_refine(w)
    g2 = run_refine(w)
    assert np.array_equal(g1, g2), "two runs must be bitwise equal"
    # user 1's rows changed: users 0 and 2 unchanged, bitwise
    X = w["X"].clone()
    X[600:900] = -X[600:900]
    g3 = run_refine(w, X=X)
    assert np.array_equal(g3[0], g1[0]) and np.array_equal(g3[2], g1[2]) and not np.array_equal(g3[1], g1[1])
    # masked rows are never read as numbers
    X = w["X"].clone()
    X[w["mask"] == 0] = float("nan")
    assert np.array_equal(run_refine(w, X=X), g1), "masked NaN rows leaked"


def test_refine_eps_and_empty_batch():
    w = W.random_refine_case(414, B=2, H=4, m=64, dh=32, lengths=[200, 70], n_layers=2)
    g = run_refine(w, eps=1e-2)
    o = oracle_refine(w, eps=1e-2)
    assert_parity(g, o, "bf16", "refine eps = 1e-2")
    e = sa.sa_refine_forward(w["X"][:0].to(device()), w["P0"].to(device()),
                             [{k: v.to(device()) for k, v in L.items()} for L in w["layers"]],
                             torch.zeros(1, dtype=torch.int32, device=device()), 4)
    assert e.shape == (0, 64, 128)
