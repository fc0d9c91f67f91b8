"""Double-precision CPU oracle for Sketch Attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.  The one module
both sides use is ``workloads`` (seeded input generators, no SA arithmetic).

The arithmetic lives in ``sa_oracle.c`` (plain C, double, two-pass softmax);
this module only builds it with gcc, loads it with ctypes and marshals arrays.
Definitions followed: SequenceO1 paper, section 3.1 (scores, prototype
normalisation display, sketch construction), appendix A.4 (the same map written
as an implicit length projection) and section 4.4 (the naive materialised
path, reproduced by :func:`assignment`).  The history-axis softmax
``S = softmax_L(P K^T * scale) V`` is the default reading; the prototype-axis
softmax of the section 3.1 display is ``norm="prototype"``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsa_oracle.so")

F32, BF16, F64 = 0, 1, 2
HISTORY, PROTOTYPE = 0, 1
_NORMS = {"history": HISTORY, "prototype": PROTOTYPE}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("m", ctypes.c_int32), ("dh", ctypes.c_int32),
        ("total_rows", ctypes.c_int64),
        ("L_max", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("k_row_stride", ctypes.c_int64), ("v_row_stride", ctypes.c_int64),
        ("p_user_stride", ctypes.c_int64),
    ]


def build(extra_flags: tuple[str, ...] = (), out: str | None = None, src: str | None = None) -> str:
    """Compile ``sa_oracle.c`` (or ``src``) into a shared library (no fast-math)
    and return its path."""
    out = out or _LIB_PATH
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
           *extra_flags, src or _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


class using:
    """Context manager: route every call of this module through the library
    at ``path`` (used by the mutation test, which plants mistakes in copies of
    the oracle and checks that the pins reject them)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(lib):
    vp, pp = ctypes.c_void_p, ctypes.POINTER(_Problem)
    lib.sao_forward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sao_forward.restype = ctypes.c_int
    lib.sao_forward_sample.argtypes = [pp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp]
    lib.sao_forward_sample.restype = ctypes.c_int
    lib.sao_assignment.argtypes = [pp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, vp]
    lib.sao_assignment.restype = ctypes.c_int64
    lib.sao_project.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_int64, vp, ctypes.c_int64, ctypes.c_int64, vp]
    lib.sao_project.restype = ctypes.c_int
    lib.sao_threads.argtypes = []
    lib.sao_threads.restype = ctypes.c_int
    return lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops may use."""
    return int(load().sao_threads())


# ---------------------------------------------------------------- marshalling
def _raw(x):
    """(contiguous numpy array, dtype code) for a torch CPU tensor or numpy array.

    bfloat16 tensors are passed as their raw 16-bit storage; the C side widens
    them exactly.
    """
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"unsupported dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _opt_int32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.int32)


def _opt_u8(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.uint8)


def _problem(P, K, cu, L_max, norm, scale, p_user_stride=0):
    """Shapes: P [H, m, dh] (or [B, H, m, dh] with per-user prototypes),
    K [rows, H, dh] (packed) or [B, L_max, H, dh] (dense)."""
    H, m, dh = P.shape[-3:]
    if cu is not None:
        rows = K.shape[0]
        B = len(cu) - 1
        Lm = 0
    else:
        B, Lm = K.shape[0], K.shape[1]
        rows = B * Lm
    pb = _Problem(B=B, H=H, m=m, dh=dh, total_rows=rows, L_max=Lm, in_dtype=0,
                  norm=_NORMS[norm], scale=float(scale or 0.0), k_row_stride=0, v_row_stride=0,
                  p_user_stride=p_user_stride)
    return pb


def forward(P, K, V, cu_offsets=None, lengths=None, mask=None, norm="history", scale=None):
    """Full SA forward in double.

    P: [H, m, dh] shared by every user, or [B, H, m, dh] with a prototype set
    per user (user b's scores use P[b]); K, V: packed [rows, H, dh] with ``cu_offsets`` [B+1], or
    dense [B, L_max, H, dh] with optional ``lengths`` [B].  ``mask``: per row
    (packed: [rows]; dense: [B, L_max]), 0 = excluded.
    Returns (S [B, H, m, dh] float64, lse): lse is [B, H, m] for the history
    axis and [rows, H] (natural log of the per-token normaliser) for the
    prototype axis.
    """
    lib = load()
    Pr, dt = _raw(P)
    Kr, dk = _raw(K)
    Vr, dv = _raw(V)
    if not (dt == dk == dv):
        raise TypeError("P, K, V must share one dtype")
    cu = _opt_int32(cu_offsets)
    ln = _opt_int32(lengths)
    mk = _opt_u8(mask)
    pb = _problem(Pr, Kr, cu, None, norm, scale, p_user_stride=_user_stride(Pr, cu, Kr))
    pb.in_dtype = dt
    S = np.zeros((pb.B, pb.H, pb.m, pb.dh), dtype=np.float64)
    if pb.norm == HISTORY:
        lse = np.zeros((pb.B, pb.H, pb.m), dtype=np.float64)
    else:
        lse = np.zeros((pb.total_rows, pb.H), dtype=np.float64)
    rc = lib.sao_forward(ctypes.byref(pb), _ptr(Pr), _ptr(Kr), _ptr(Vr), _ptr(cu), _ptr(ln), _ptr(mk),
                         _ptr(S), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return S, lse


def _user_stride(Pr, cu, Kr):
    """p_user_stride of the C problem: 0 for shared P [H, m, dh], H*m*dh for
    per-user P [B, H, m, dh] (which must have one set per user)."""
    if Pr.ndim == 3:
        return 0
    if Pr.ndim != 4:
        raise ValueError("P must be [H, m, dh] or [B, H, m, dh]")
    B = len(cu) - 1 if cu is not None else Kr.shape[0]
    if Pr.shape[0] != B:
        raise ValueError(f"per-user P has {Pr.shape[0]} sets for {B} users")
    return int(Pr.shape[1] * Pr.shape[2] * Pr.shape[3])


def forward_sample(P, K, V, bhj, cu_offsets=None, lengths=None, mask=None, scale=None):
    """History axis: rows S[b, h, j, :] for each (b, h, j) in ``bhj`` -> ([n, dh], lse [n])."""
    lib = load()
    Pr, dt = _raw(P)
    Kr, _ = _raw(K)
    Vr, _ = _raw(V)
    cu = _opt_int32(cu_offsets)
    ln = _opt_int32(lengths)
    mk = _opt_u8(mask)
    pb = _problem(Pr, Kr, cu, None, "history", scale, p_user_stride=_user_stride(Pr, cu, Kr))
    pb.in_dtype = dt
    idx = np.ascontiguousarray(np.asarray(bhj, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((idx.shape[0], pb.dh), dtype=np.float64)
    lse = np.zeros((idx.shape[0],), dtype=np.float64)
    rc = lib.sao_forward_sample(ctypes.byref(pb), _ptr(Pr), _ptr(Kr), _ptr(Vr), _ptr(cu), _ptr(ln), _ptr(mk),
                                idx.shape[0], _ptr(idx), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out, lse


def assignment(P, K, b, h, cu_offsets=None, lengths=None, mask=None, norm="history", scale=None):
    """The materialised assignment matrix A [m, n_valid] of user b, head h."""
    lib = load()
    Pr, dt = _raw(P)
    Kr, _ = _raw(K)
    cu = _opt_int32(cu_offsets)
    ln = _opt_int32(lengths)
    mk = _opt_u8(mask)
    pb = _problem(Pr, Kr, cu, None, norm, scale)
    pb.in_dtype = dt
    cap = pb.total_rows if cu is not None else pb.L_max
    cap = max(int(cap), 1)
    A = np.zeros((pb.m, cap), dtype=np.float64)
    n = lib.sao_assignment(ctypes.byref(pb), _ptr(Pr), _ptr(Kr), _ptr(cu), _ptr(ln), _ptr(mk),
                           int(b), int(h), cap, _ptr(A))
    if n < 0:
        raise ValueError("oracle rejected the problem")
    return A[:, :n].copy()


def project(X, W, rows=None, c0=0, nc=None):
    """out[r, c] = sum_k X[rows[r], k] * W[k, c0 + c] in double (no rounding)."""
    lib = load()
    Xr, dx = _raw(X)
    Wr, dw = _raw(W)
    if dx != dw:
        raise TypeError("X and W must share one dtype")
    d_model = Xr.shape[-1]
    ldw = Wr.shape[1]
    nc = ldw - c0 if nc is None else nc
    if rows is None:
        nrows = Xr.shape[0]
        rr = None
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rr.shape[0]
    out = np.zeros((nrows, nc), dtype=np.float64)
    lib.sao_project(_ptr(Xr), _ptr(Wr), dx, d_model, ldw, nrows, _ptr(rr), c0, nc, _ptr(out))
    return out


def fused_forward(X, Wk, Wv, P, cu_offsets, mask=None, norm="history", scale=None):
    """Fused-projection forward: K = X Wk and V = X Wv in double (V = X when
    ``Wv`` is None), then the SA forward on the exact products."""
    Kd = project(X, Wk)
    Vd = project(X, Wv) if Wv is not None else _widen64(X)
    Pd = _widen64(P)
    H, m, dh = Pd.shape
    rows = Kd.shape[0]
    return forward(Pd, Kd.reshape(rows, H, dh), Vd.reshape(rows, H, dh), cu_offsets=cu_offsets,
                   mask=mask, norm=norm, scale=scale)


def fused_forward_sample(X, Wk, Wv, P, cu_offsets, bhj, mask=None, scale=None):
    """History axis, sampled (b, h, j) rows of the fused-projection forward."""
    Pd = _widen64(P)
    H, m, dh = Pd.shape
    cu = _opt_int32(cu_offsets)
    out = np.zeros((len(bhj), dh))
    lse = np.zeros((len(bhj),))
    for t, (b, h, j) in enumerate(bhj):
        rows = np.arange(cu[b], cu[b + 1], dtype=np.int64)
        Kd = project(X, Wk, rows=rows, c0=h * dh, nc=dh)
        Vd = project(X, Wv, rows=rows, c0=h * dh, nc=dh) if Wv is not None else _widen64(X)[rows, h * dh:(h + 1) * dh]
        mk = None if mask is None else _opt_u8(mask)[cu[b]:cu[b + 1]]
        o, l = forward_sample(Pd[h:h + 1, j:j + 1], Kd.reshape(-1, 1, dh), Vd.reshape(-1, 1, dh), [(0, 0, 0)],
                              cu_offsets=np.array([0, len(rows)], dtype=np.int32), mask=mk, scale=scale)
        out[t] = o[0]
        lse[t] = l[0]
    return out, lse


def _widen64(x):
    a, d = _raw(x)
    if d == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


widen64 = _widen64
