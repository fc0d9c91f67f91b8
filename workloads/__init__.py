"""Seeded synthetic inputs for Sketch Attention workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  It is the one module that both the GPU path's tests and
the CPU oracle consume, so that both see the very same stored tensors.

Recipe (every workload): ``numpy.random.SeedSequence(seed)`` spawns child
streams in a fixed order -- [lengths, prototypes, extra (per-user means or the
projection weights), user 0, user 1, ...] -- each driving a PCG64
``Generator``.  Normal draws are float32 ``standard_normal``; bf16 tensors are
the float32 draws rounded to nearest-even by ``torch.Tensor.to(bfloat16)``.
Each user's rows come from that user's own stream (keys first, then values,
or the raw embeddings X), so a user's data does not depend on the others.

The five named workloads mirror the shapes the SequenceO1 paper works at:
histories of up to 100K interactions per user (section 2.1), a recent 10K
suffix (section 3.4), hundreds of prototypes (section 1), and d = 128-wide
behaviour embeddings (table 2).  The paper measures on a proprietary Douyin
dataset; these seeded draws stand in for it.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np


@dataclasses.dataclass
class Spec:
    name: str
    B: int
    H: int
    m: int
    dh: int
    dtype: str              # "f32" or "bf16"
    layout: str             # "dense" or "packed"
    lengths: str            # "fixed", "loguniform", "lognormal"
    L: int = 0              # fixed length
    L_lo: int = 0
    L_hi: int = 0
    L_median: float = 0.0
    sigma: float = 0.0
    ones: tuple = ()        # users forced to length 1
    mean_offset_var: float = 0.0   # per-user per-channel mean offset on K (variance)
    d_model: int = 0        # > 0: fused projection workload (X, Wk, Wv)
    w_var: float = 0.0      # variance of projection weights
    seed: int = 0


SPECS = {
    1: Spec("tiny_fp32", B=1, H=1, m=16, dh=32, dtype="f32", layout="dense", lengths="fixed", L=1000, seed=1),
    2: Spec("suffix10k_bf16", B=32, H=4, m=64, dh=32, dtype="bf16", layout="dense", lengths="fixed", L=10000, seed=2),
    3: Spec("varlen_bf16", B=64, H=4, m=64, dh=32, dtype="bf16", layout="packed", lengths="loguniform",
            L_lo=1000, L_hi=100000, ones=(0, 21, 42, 63), seed=3),
    4: Spec("full100k_bf16", B=16, H=8, m=128, dh=64, dtype="bf16", layout="packed", lengths="fixed", L=100000,
            mean_offset_var=0.5, seed=4),
    5: Spec("fusedproj_bf16", B=128, H=8, m=256, dh=32, dtype="bf16", layout="packed", lengths="lognormal",
            L_median=20000.0, sigma=1.0, L_lo=100, L_hi=100000, d_model=256, w_var=1.0 / 256, seed=5),
}


def draw_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    if spec.lengths == "fixed":
        L = np.full(spec.B, spec.L, dtype=np.int64)
    elif spec.lengths == "loguniform":
        u = rng.uniform(math.log(spec.L_lo), math.log(spec.L_hi), size=spec.B)
        L = np.rint(np.exp(u)).astype(np.int64)          # rint: round half to even
    elif spec.lengths == "lognormal":
        z = rng.standard_normal(spec.B)
        L = np.clip(np.rint(np.exp(math.log(spec.L_median) + spec.sigma * z)), spec.L_lo, spec.L_hi).astype(np.int64)
    else:
        raise ValueError(spec.lengths)
    for b in spec.ones:
        if b < spec.B:
            L[b] = 1
    return L


def _to_torch(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make(cfg, *, B: int | None = None, max_len: int | None = None, seed: int | None = None,
         threads: int = 8, dtype: str | None = None, layout: str | None = None):
    """Draw a workload.  ``cfg`` is a workload number (1-5) or a :class:`Spec`.

    ``B`` / ``max_len`` shrink the workload (fewer users, lengths capped) while
    keeping its distribution: the first B users' streams and lengths are the
    same as in the full workload.  Returns a dict of CPU torch tensors:
      P [H, m, dh]; lengths [B] (int32); and either
      K, V packed [rows, H, dh] with cu_offsets [B+1] (int32), or
      K, V dense [B, L_max, H, dh] (rows past a user's length are zero), or,
      for the fused-projection workload, X [rows, d_model], Wk, Wv [d_model, H*dh]
      with cu_offsets.
    """
    import torch
    spec = SPECS[cfg] if isinstance(cfg, int) else cfg
    spec = dataclasses.replace(spec)
    dt = dtype or spec.dtype
    lay = layout or spec.layout
    seed = spec.seed if seed is None else seed
    Bfull = spec.B
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(3 + Bfull)
    g_len, g_p, g_extra = (np.random.Generator(np.random.PCG64(k)) for k in kids[:3])
    lengths = draw_lengths(spec, g_len)
    if B is not None and B > Bfull:
        raise ValueError(f"workload {spec.name} has {Bfull} users; asked for {B}")
    nb = Bfull if B is None else B
    lengths = lengths[:nb].copy()
    if max_len is not None:
        lengths = np.minimum(lengths, max_len)
    H, m, dh = spec.H, spec.m, spec.dh
    P = g_p.standard_normal((H, m, dh), dtype=np.float32)
    out = {"spec": spec, "B": nb, "H": H, "m": m, "dh": dh, "dtype": dt, "layout": lay,
           "lengths": torch.from_numpy(lengths.astype(np.int32)), "P": _to_torch(P, dt)}
    user_seeds = kids[3:3 + nb]

    if spec.d_model:
        dm = spec.d_model
        std = math.sqrt(spec.w_var)
        Wk = g_extra.standard_normal((dm, H * dh), dtype=np.float32) * np.float32(std)
        Wv = g_extra.standard_normal((dm, H * dh), dtype=np.float32) * np.float32(std)
        out["Wk"], out["Wv"] = _to_torch(Wk, dt), _to_torch(Wv, dt)
        cu = np.zeros(nb + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lengths)
        X = torch.empty((int(cu[-1]), dm), dtype=torch.bfloat16 if dt == "bf16" else torch.float32)

        def fill_x(b):
            g = np.random.Generator(np.random.PCG64(user_seeds[b]))
            X[cu[b]:cu[b + 1]] = _to_torch(g.standard_normal((int(lengths[b]), dm), dtype=np.float32), dt)

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill_x, range(nb)))
        out["X"] = X
        out["cu_offsets"] = torch.from_numpy(cu.astype(np.int32))
        out["d_model"] = dm
        return out

    mu = None
    if spec.mean_offset_var > 0:
        mu = g_extra.standard_normal((Bfull, H, dh), dtype=np.float32) * np.float32(math.sqrt(spec.mean_offset_var))

    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    if lay == "packed":
        cu = np.zeros(nb + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lengths)
        rows = int(cu[-1])
        K = torch.empty((rows, H, dh), dtype=tdt)
        V = torch.empty((rows, H, dh), dtype=tdt)
        out["cu_offsets"] = torch.from_numpy(cu.astype(np.int32))
    else:
        Lmax = int(lengths.max()) if nb else 0
        K = torch.zeros((nb, Lmax, H, dh), dtype=tdt)
        V = torch.zeros((nb, Lmax, H, dh), dtype=tdt)

    def fill(b):
        g = np.random.Generator(np.random.PCG64(user_seeds[b]))
        n = int(lengths[b])
        k = g.standard_normal((n, H, dh), dtype=np.float32)
        if mu is not None:
            k += mu[b][None]
        v = g.standard_normal((n, H, dh), dtype=np.float32)
        if lay == "packed":
            K[cu[b]:cu[b + 1]] = _to_torch(k, dt)
            V[cu[b]:cu[b + 1]] = _to_torch(v, dt)
        else:
            K[b, :n] = _to_torch(k, dt)
            V[b, :n] = _to_torch(v, dt)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(nb)))
    out["K"], out["V"] = K, V
    return out


def random_case(seed: int, *, B: int, H: int, m: int, dh: int, lengths, dtype: str = "f32",
                layout: str = "packed", mask_p: float = 0.0, std: float = 1.0):
    """A small free-form case (same recipe, explicit sizes) for edge-case tests.

    ``lengths``: list of per-user lengths.  ``mask_p`` > 0 adds a per-row mask
    with that drop probability.  Returns the same dict layout as :func:`make`
    (plus ``mask`` when requested).
    """
    import torch
    spec = Spec("case", B=B, H=H, m=m, dh=dh, dtype=dtype, layout=layout, lengths="fixed", seed=seed)
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(3 + B)
    g_p = np.random.Generator(np.random.PCG64(kids[1]))
    g_mask = np.random.Generator(np.random.PCG64(kids[2]))
    lengths = np.asarray(lengths, dtype=np.int64)
    P = g_p.standard_normal((H, m, dh), dtype=np.float32) * np.float32(std)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {"spec": spec, "B": B, "H": H, "m": m, "dh": dh, "dtype": dtype, "layout": layout,
           "lengths": torch.from_numpy(lengths.astype(np.int32)), "P": _to_torch(P, dtype)}
    if layout == "packed":
        cu = np.zeros(B + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lengths)
        rows = int(cu[-1])
        K = torch.zeros((rows, H, dh), dtype=tdt)
        V = torch.zeros((rows, H, dh), dtype=tdt)
        out["cu_offsets"] = torch.from_numpy(cu.astype(np.int32))
        nrows_mask = rows
    else:
        Lmax = int(lengths.max()) if B else 0
        K = torch.zeros((B, Lmax, H, dh), dtype=tdt)
        V = torch.zeros((B, Lmax, H, dh), dtype=tdt)
        nrows_mask = B * Lmax
    for b in range(B):
        g = np.random.Generator(np.random.PCG64(kids[3 + b]))
        n = int(lengths[b])
        k = _to_torch(g.standard_normal((n, H, dh), dtype=np.float32) * np.float32(std), dtype)
        v = _to_torch(g.standard_normal((n, H, dh), dtype=np.float32), dtype)
        if layout == "packed":
            K[out["cu_offsets"][b]:out["cu_offsets"][b + 1]] = k
            V[out["cu_offsets"][b]:out["cu_offsets"][b + 1]] = v
        else:
            K[b, :n] = k
            V[b, :n] = v
    out["K"], out["V"] = K, V
    if mask_p > 0:
        mk = (g_mask.uniform(size=nrows_mask) >= mask_p).astype(np.uint8)
        out["mask"] = torch.from_numpy(mk) if layout == "packed" else torch.from_numpy(mk.reshape(B, -1))
    return out


def random_fused_case(seed: int, *, B: int, H: int, m: int, dh: int, d_model: int, lengths,
                      w_var: float = 1.0 / 256, mask_p: float = 0.0, per_user_p: bool = False):
    """A small free-form case of the fused-projection recipe (bf16): X rows
    ~ N(0, 1) [rows, d_model], Wk, Wv ~ N(0, w_var) [d_model, H*dh], P ~ N(0, 1)
    [H, m, dh] (or [B, H, m, dh] with ``per_user_p``), packed by ``lengths``;
    ``mask_p`` > 0 adds a per-row mask with that drop probability."""
    import torch
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(3 + B)
    g_p, g_w, g_mask = (np.random.Generator(np.random.PCG64(k)) for k in kids[:3])
    lengths = np.asarray(lengths, dtype=np.int64)
    pshape = (B, H, m, dh) if per_user_p else (H, m, dh)
    P = g_p.standard_normal(pshape, dtype=np.float32)
    std = np.float32(math.sqrt(w_var))
    Wk = g_w.standard_normal((d_model, H * dh), dtype=np.float32) * std
    Wv = g_w.standard_normal((d_model, H * dh), dtype=np.float32) * std
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    X = torch.empty((int(cu[-1]), d_model), dtype=torch.bfloat16)
    for b in range(B):
        g = np.random.Generator(np.random.PCG64(kids[3 + b]))
        X[cu[b]:cu[b + 1]] = _to_torch(g.standard_normal((int(lengths[b]), d_model), dtype=np.float32), "bf16")
    spec = Spec("fused_case", B=B, H=H, m=m, dh=dh, dtype="bf16", layout="packed", lengths="fixed", seed=seed,
                d_model=d_model)
    out = {"spec": spec, "B": B, "H": H, "m": m, "dh": dh, "dtype": "bf16", "layout": "packed",
           "lengths": torch.from_numpy(lengths.astype(np.int32)), "P": _to_torch(P, "bf16"),
           "Wk": _to_torch(Wk, "bf16"), "Wv": _to_torch(Wv, "bf16"), "X": X,
           "cu_offsets": torch.from_numpy(cu.astype(np.int32)), "d_model": d_model}
    if mask_p > 0:
        out["mask"] = torch.from_numpy((g_mask.uniform(size=int(cu[-1])) >= mask_p).astype(np.uint8))
    return out


def refine_layers(seed: int, d: int, n_layers: int):
    """Seeded weights of stacked refinement layers (random init, no training):
    Wq, Wk, W1, W3 ~ N(0, 1/d) and W2 ~ N(0, 1/(2d)) in bf16 ([in, out]),
    layer-norm gains 1 + N(0, 0.01) and biases N(0, 0.01) in fp32.  The
    1/fan-in variances keep queries, keys and FFN outputs at unit scale."""
    import torch
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7919])))
    out = []
    for _ in range(n_layers):
        L = {}
        for k, shape, var in (("Wq", (d, d), 1.0 / d), ("Wk", (d, d), 1.0 / d), ("W1", (d, 2 * d), 1.0 / d),
                              ("W3", (d, 2 * d), 1.0 / d), ("W2", (2 * d, d), 0.5 / d)):
            L[k] = _to_torch(g.standard_normal(shape, dtype=np.float32) * np.float32(math.sqrt(var)), "bf16")
        for k in ("ln1", "ln2"):
            L[k + "_g"] = torch.from_numpy(1 + 0.1 * g.standard_normal(d, dtype=np.float32))
            L[k + "_b"] = torch.from_numpy(0.1 * g.standard_normal(d, dtype=np.float32))
        out.append(L)
    return out


def random_refine_case(seed: int, *, B: int, H: int, m: int, dh: int, lengths, n_layers: int = 2,
                       mask_p: float = 0.0):
    """Stacked-refinement inputs: the fused-projection recipe's X (N(0, 1)
    bf16 rows, d = H*dh, packed by ``lengths``), prototypes P0 ~ N(0, 1)
    [m, d] fp32 and ``n_layers`` seeded layers (:func:`refine_layers`)."""
    import torch
    d = H * dh
    w = random_fused_case(seed, B=B, H=H, m=m, dh=dh, d_model=d, lengths=lengths, mask_p=mask_p)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 104729])))
    w["P0"] = torch.from_numpy(g.standard_normal((m, d), dtype=np.float32))
    w["layers"] = refine_layers(seed, d, n_layers)
    for k in ("P", "Wk", "Wv"):
        del w[k]
    return w


def random_stca_case(seed: int, *, lengths, targets, D: int = 1024, h: int = 16, windows: str | None = None):
    """Inputs of STCA single-query attention (bf16): history rows X ~ N(0, 1)
    [rows, D] packed by ``lengths`` (the adapted sketch, or a recent suffix),
    target vectors xt ~ N(0, 1) [T, D] grouped by user with ``targets`` per
    user, and W_Q, W_K, W_V ~ N(0, 1/D) [D, D] (unit-scale projections, so
    the scaled scores are about unit-scale too).  ``windows``: None (every
    target sees its user's rows), "random" (a uniform [lo, hi) per target,
    empty ones included) or "requests" (a user's targets, in order, fall in
    four equal groups, some possibly empty, standing for four requests;
    group r sees the first (r+1)/4 of the user's rows).  Windows are int32 [T, 2], relative to the user's first
    row."""
    import torch
    ss = np.random.SeedSequence([seed, 15485863])
    kids = ss.spawn(3 + len(lengths))
    g_t, g_w, g_win = (np.random.Generator(np.random.PCG64(k)) for k in kids[:3])
    lengths = np.asarray(lengths, dtype=np.int64)
    targets = np.asarray(targets, dtype=np.int64)
    B = len(lengths)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    tcu = np.zeros(B + 1, dtype=np.int64)
    tcu[1:] = np.cumsum(targets)
    T = int(tcu[-1])
    std = np.float32(1.0 / math.sqrt(D))
    W = [_to_torch(g_w.standard_normal((D, D), dtype=np.float32) * std, "bf16") for _ in range(3)]
    xt = _to_torch(g_t.standard_normal((T, D), dtype=np.float32), "bf16")
    X = torch.empty((int(cu[-1]), D), dtype=torch.bfloat16)
    for b in range(B):
        g = np.random.Generator(np.random.PCG64(kids[3 + b]))
        X[cu[b]:cu[b + 1]] = _to_torch(g.standard_normal((int(lengths[b]), D), dtype=np.float32), "bf16")
    out = {"B": B, "D": D, "h": h, "T": T, "xt": xt, "X": X, "Wq": W[0], "Wk": W[1], "Wv": W[2],
           "lengths": torch.from_numpy(lengths.astype(np.int32)), "targets": torch.from_numpy(targets.astype(np.int32)),
           "cu_offsets": torch.from_numpy(cu.astype(np.int32)), "t_offsets": torch.from_numpy(tcu.astype(np.int32)),
           "windows": None}
    if windows is not None:
        win = np.zeros((T, 2), dtype=np.int32)
        for b in range(B):
            n, t0, nt = int(lengths[b]), int(tcu[b]), int(targets[b])
            for k in range(nt):
                if windows == "random":
                    lo = int(g_win.integers(0, n + 1))
                    win[t0 + k] = (lo, int(g_win.integers(lo, n + 1)))
                else:
                    r = 4 * k // nt
                    win[t0 + k] = (0, (n * (r + 1)) // 4)
        out["windows"] = torch.from_numpy(win)
    return out


def algorithmic_bytes(w: dict) -> int:
    """HBM bytes one forward must move at minimum: K and V (or X and the two
    projection matrices), the prototypes, the fp32 sketch and the offsets."""
    el = 2 if w["dtype"] == "bf16" else 4
    H, m, dh, B = w["H"], w["m"], w["dh"], w["B"]
    total = int(w["lengths"].sum())
    if "X" in w:
        dm = w["d_model"]
        n = total * dm * el + 2 * dm * H * dh * el
    else:
        n = 2 * total * H * dh * el
    n += H * m * dh * el + B * H * m * dh * 4 + 4 * (B + 1)
    return n
