"""Helpers shared by the GPU tests: move a seeded workload to the device, run
the library through its C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import sketch_attention_flashsa_amd as sa

# Parity bars: fp32 inputs -> max |g - o| / max |o| <= 1e-5 over the output;
# bf16 inputs -> relative L2 error <= 1e-2 over the output, oracle fed the
# same bf16 tensors, and every output row (last axis: one (user, head,
# prototype) sketch row, one target's output, one gradient row) within a
# relative L2 error of 5e-2 on its own, so that one wrong row cannot hide in
# a large output.  Rows the oracle gives as exactly zero have no relative
# error; the tests whose contract makes them exactly zero (empty users) assert
# that directly, and others (a single-row user's key gradient, zero only by
# the cancellation of two terms) are left to the global bar.
TOL_F32 = 1e-5
TOL_BF16 = 1e-2
ROW_TOL_BF16 = 5e-2


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def to_dev(w: dict, dev=None) -> dict:
    dev = dev or device()
    out = {}
    for k, v in w.items():
        out[k] = v.to(dev) if isinstance(v, torch.Tensor) else v
    return out


def run(w: dict, norm="history", mask=None, lengths=None, use_lengths=True, **kw):
    """Run sa_forward on the GPU for a workload dict (CPU tensors); returns
    (S, lse) as float64 numpy arrays."""
    dev = device()
    d = to_dev(w, dev)
    msk = mask if mask is not None else w.get("mask")
    msk = None if msk is None else msk.to(dev)
    if w["layout"] == "packed":
        S, lse = sa.sa_forward(d["P"], d["K"], d["V"], cu_offsets=d["cu_offsets"], mask=msk, norm=norm,
                               return_lse=True, **kw)
    else:
        ln = lengths if lengths is not None else (d["lengths"] if use_lengths else None)
        S, lse = sa.sa_forward(d["P"], d["K"], d["V"], lengths=None if ln is None else ln.to(dev), mask=msk,
                               norm=norm, return_lse=True, **kw)
    torch.cuda.synchronize()
    return S.double().cpu().numpy(), lse.double().cpu().numpy()


def rel_l2(g, o):
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    den = np.linalg.norm(o.ravel())
    return float(np.linalg.norm((g - o).ravel()) / (den if den > 0 else 1.0))


def rel_inf(g, o):
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    den = np.max(np.abs(o)) if o.size else 1.0
    return float(np.max(np.abs(g - o)) / (den if den > 0 else 1.0)) if o.size else 0.0


def row_rel_l2(g, o):
    """Relative L2 error of every row (last axis) and the rows' oracle norms."""
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    n = o.shape[-1] if o.ndim else 1
    g2, o2 = g.reshape(-1, n), o.reshape(-1, n)
    den = np.linalg.norm(o2, axis=1)
    num = np.linalg.norm(g2 - o2, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num), den


def assert_parity(g, o, dtype, what="", row_tol=ROW_TOL_BF16):
    if dtype == "f32":
        e = rel_inf(g, o)
        assert e <= TOL_F32, f"{what}: fp32 max relative error {e:.3e} > {TOL_F32}"
    else:
        e = rel_l2(g, o)
        assert e <= TOL_BF16, f"{what}: bf16 relative L2 error {e:.3e} > {TOL_BF16}"
        if row_tol is not None and np.asarray(o).size:
            r, den = row_rel_l2(g, o)
            zero = den == 0
            worst = int(np.argmax(np.where(zero, 0.0, r)))
            assert r[worst] <= row_tol or zero[worst], \
                f"{what}: row {worst} relative L2 error {r[worst]:.3e} > {row_tol} (whole output {e:.3e})"
    return e


def assert_lse(g, o, dtype, what=""):
    fin = np.isfinite(o)
    assert np.array_equal(fin, np.isfinite(g)), f"{what}: -inf pattern of lse differs"
    tol = 1e-4 if dtype == "f32" else 2e-2
    err = float(np.max(np.abs(g[fin] - o[fin]), initial=0.0))
    assert err <= tol, f"{what}: lse abs error {err:.3e} > {tol}"
    return err
