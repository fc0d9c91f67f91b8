"""Python binding of libsketchattn (Sketch Attention on MI355X / gfx950).

A thin ctypes layer over the C ABI declared in ``include/sketchattn.h``: it
checks torch tensors, allocates outputs and the workspace with torch, and
passes raw device pointers and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is not built this module raises on import of the compute functions.

Names follow the C ABI: :func:`sa_forward`, :func:`sa_forward_fused_proj`,
:func:`sa_forward_workspace_size`, :func:`sa_status_string`,
:func:`sa_last_error`, :func:`sa_version`.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsketchattn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
SA_DTYPE_F32, SA_DTYPE_BF16 = 0, 1
SA_NORM_HISTORY, SA_NORM_PROTOTYPE = 0, 1
SA_FLAG_BF16_GRADS = 1
SA_FLAG_CHECK_OFFSETS = 2
_NORMS = {"history": SA_NORM_HISTORY, "prototype": SA_NORM_PROTOTYPE}

EXPORTED = ("sa_forward", "sa_forward_workspace_size", "sa_forward_noalloc", "sa_forward_noalloc_max_workspace",
            "sa_forward_kernel_name", "sa_forward_fused_proj",
            "sa_forward_fused_proj_workspace_size", "sa_refine_forward", "sa_refine_workspace_size",
            "sa_backward", "sa_backward_workspace_size", "sa_stca_attention", "sa_stca_workspace_size",
            "sa_set_timing_events", "sa_set_tuning", "sa_check_offsets_host", "sa_status_string", "sa_last_error",
            "sa_version")


class SaRefineLayer(ctypes.Structure):
    """Mirror of ``sa_refine_layer`` in include/sketchattn.h."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("Wq", "Wk", "ln1_g", "ln1_b", "W1", "W3", "W2", "ln2_g", "ln2_b")]


class SaProblem(ctypes.Structure):
    """Mirror of ``sa_problem`` in include/sketchattn.h."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("m", ctypes.c_int32), ("dh", ctypes.c_int32),
        ("total_rows", ctypes.c_int64),
        ("L_max", ctypes.c_int32), ("dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("k_row_stride", ctypes.c_int64), ("v_row_stride", ctypes.c_int64),
        ("q_batch_stride", ctypes.c_int64),
        ("chunk_rows", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


class SaTuning(ctypes.Structure):
    """Mirror of ``sa_tuning`` in include/sketchattn.h (0 = the default)."""
    _fields_ = [(n, ctypes.c_int32) for n in ("register_staged", "stream_waves", "blocks_per_cu", "range_split",
                                              "bf16_tile_mb", "bf16_tile_nw", "bwd_blocks_per_cu",
                                              "bwd_dp_register_staged")]


class SaStcaProblem(ctypes.Structure):
    """Mirror of ``sa_stca_problem`` in include/sketchattn.h."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("h", ctypes.c_int32),
        ("total_rows", ctypes.c_int64), ("x_row_stride", ctypes.c_int64), ("scale", ctypes.c_float),
        ("flags", ctypes.c_int32),
    ]


class SketchAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{sa_status_string(status)}: {detail}")
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load libsketchattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libsketchattn.so not found at {p}; run `python -m sketch_attention_flashsa_amd.build`")
    lib = ctypes.CDLL(p)
    vp, pp = ctypes.c_void_p, ctypes.POINTER(SaProblem)
    lib.sa_forward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_forward.restype = ctypes.c_int
    lib.sa_forward_workspace_size.argtypes = [pp]
    lib.sa_forward_workspace_size.restype = ctypes.c_size_t
    lib.sa_forward_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sa_forward_noalloc.restype = ctypes.c_int
    lib.sa_forward_noalloc_max_workspace.argtypes = []
    lib.sa_forward_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.sa_forward_kernel_name.argtypes = [pp]
    lib.sa_forward_kernel_name.restype = ctypes.c_char_p
    lib.sa_forward_fused_proj.argtypes = [pp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_forward_fused_proj.restype = ctypes.c_int
    lib.sa_forward_fused_proj_workspace_size.argtypes = [pp, ctypes.c_int32]
    lib.sa_forward_fused_proj_workspace_size.restype = ctypes.c_size_t
    lib.sa_refine_forward.argtypes = [pp, vp, ctypes.c_int32, vp, ctypes.c_int32, ctypes.POINTER(SaRefineLayer),
                                      ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_refine_forward.restype = ctypes.c_int
    lib.sa_backward.argtypes = [pp] + [vp] * 13 + [ctypes.c_size_t, vp]
    lib.sa_backward.restype = ctypes.c_int
    lib.sa_backward_workspace_size.argtypes = [pp]
    lib.sa_backward_workspace_size.restype = ctypes.c_size_t
    lib.sa_refine_workspace_size.argtypes = [pp, ctypes.c_int32, ctypes.c_int32]
    lib.sa_refine_workspace_size.restype = ctypes.c_size_t
    sp = ctypes.POINTER(SaStcaProblem)
    lib.sa_stca_attention.argtypes = [sp] + [vp] * 10 + [ctypes.c_size_t, vp]
    lib.sa_stca_attention.restype = ctypes.c_int
    lib.sa_stca_workspace_size.argtypes = [sp]
    lib.sa_stca_workspace_size.restype = ctypes.c_size_t
    lib.sa_status_string.argtypes = [ctypes.c_int32]
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_last_error.argtypes = []
    lib.sa_last_error.restype = ctypes.c_char_p
    lib.sa_version.argtypes = []
    lib.sa_version.restype = ctypes.c_int
    lib.sa_set_timing_events.argtypes = [vp, vp]
    lib.sa_set_timing_events.restype = ctypes.c_int
    lib.sa_set_tuning.argtypes = [ctypes.POINTER(SaTuning)]
    lib.sa_set_tuning.restype = ctypes.c_int
    lib.sa_check_offsets_host.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)]
    lib.sa_check_offsets_host.restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def sa_set_timing_events(start, stop) -> None:
    """Record HIP events ``start``/``stop`` (raw hipEvent_t handles, or None)
    around the streaming kernel of the next forward call on this thread."""
    _check(load_library().sa_set_timing_events(start, stop))


def sa_set_tuning(**fields) -> None:
    """Work-split tuning for the calls this thread makes (``sa_tuning``
    fields as keywords; no keywords restores the defaults)."""
    lib = load_library()
    if not fields:
        _check(lib.sa_set_tuning(None))
        return
    t = SaTuning()
    for k, v in fields.items():
        if k not in dict(SaTuning._fields_):
            raise TypeError(f"unknown tuning field {k!r}")
        setattr(t, k, int(v))
    _check(lib.sa_set_tuning(ctypes.byref(t)))


def sa_check_offsets_host(cu_offsets, total_rows: int):
    """The offsets rules on host memory: returns (status bits, first bad
    index or -1) for an int32 sequence of B+1 offsets."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_offsets), dtype=np.int32)
    first = ctypes.c_int32(0)
    bits = load_library().sa_check_offsets_host(cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1, int(total_rows),
                                                ctypes.byref(first))
    return int(bits), int(first.value)


def sa_status_string(status: int) -> str:
    return load_library().sa_status_string(int(status)).decode()


def sa_last_error() -> str:
    return load_library().sa_last_error().decode()


def sa_version() -> int:
    return int(load_library().sa_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_problem(B, H, m, dh, total_rows, L_max=0, dtype="bf16", norm="history", scale=0.0,
                 k_row_stride=0, v_row_stride=0, q_batch_stride=0, chunk_rows=0, flags=0) -> SaProblem:
    return SaProblem(B=B, H=H, m=m, dh=dh, total_rows=total_rows, L_max=L_max,
                     dtype=SA_DTYPE_BF16 if dtype == "bf16" else SA_DTYPE_F32,
                     norm=_NORMS[norm], scale=float(scale or 0.0), k_row_stride=k_row_stride,
                     v_row_stride=v_row_stride, q_batch_stride=q_batch_stride, chunk_rows=chunk_rows, flags=flags)


def sa_forward_workspace_size(pb: SaProblem) -> int:
    return int(load_library().sa_forward_workspace_size(ctypes.byref(pb)))


def sa_forward_kernel_name(pb: SaProblem) -> str:
    """Name of the kernel that makes the pass over K/V for this problem."""
    name = load_library().sa_forward_kernel_name(ctypes.byref(pb))
    if name is None:
        raise SketchAttnError(SA_ERR_INVALID_ARG, sa_last_error())
    return name.decode()


def _check(status):
    if status != SA_OK:
        raise SketchAttnError(status, sa_last_error())


def _dtype_name(t):
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def sa_forward(P, K, V, cu_offsets=None, lengths=None, mask=None, norm: str = "history",
               return_lse: bool = False, scale: float | None = None, chunk_rows: int = 0,
               workspace=None, out=None, check_offsets: bool = False):
    """Sketch Attention forward on the GPU.

    P: [H, m, dh] (or [B, H, m, dh] per-user prototypes), bf16 or fp32.
    K, V: packed [rows, H, dh] with ``cu_offsets`` int32 [B+1], or dense
    [B, L_max, H, dh] (``cu_offsets`` None) with optional ``lengths`` int32 [B].
    ``mask``: uint8/bool per buffer row ([rows] or [B, L_max]), 0 = excluded.
    Returns S [B, H, m, dh] float32, and lse when ``return_lse``
    ([B, H, m] history axis; [rows, H] prototype axis).
    ``check_offsets`` sets SA_FLAG_CHECK_OFFSETS: the offsets are validated
    on the device and the verdict lands in ``workspace[:8]`` (int32 status,
    int32 first bad index); pass ``workspace`` to read it.
    """
    import torch
    lib = load_library()
    dt = _dtype_name(K)
    if P.dtype != K.dtype or V.dtype != K.dtype:
        raise TypeError("P, K and V must share one dtype")
    dev = K.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for name, t in (("P", P), ("K", K), ("V", V)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    per_user = P.dim() == 4
    H, m, dh = P.shape[-3:]
    if cu_offsets is not None:
        if K.dim() != 3 or K.shape[1:] != (H, dh) or V.shape != K.shape:
            raise ValueError(f"packed K/V must be [rows, {H}, {dh}]; got {tuple(K.shape)}, {tuple(V.shape)}")
        if cu_offsets.dtype != torch.int32 or cu_offsets.device != dev or cu_offsets.dim() != 1:
            raise ValueError("cu_offsets must be a 1-D int32 tensor on the same device")
        if lengths is not None:
            raise ValueError("lengths is only valid for the dense layout")
        B = cu_offsets.numel() - 1
        rows, L_max = K.shape[0], 0
    else:
        if K.dim() != 4 or K.shape[2:] != (H, dh) or V.shape != K.shape:
            raise ValueError(f"dense K/V must be [B, L_max, {H}, {dh}]; got {tuple(K.shape)}")
        B, L_max = K.shape[0], K.shape[1]
        rows = B * L_max
        if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() != B or lengths.device != dev):
            raise ValueError("lengths must be an int32 tensor [B] on the same device")
    if per_user and P.shape[0] != B:
        raise ValueError("per-user P must be [B, H, m, dh]")
    # rows must be contiguous in dh and heads; the row stride may be larger
    ks = K.stride(-3) if cu_offsets is not None else K.stride(1)
    vs = V.stride(-3) if cu_offsets is not None else V.stride(1)
    for t in (K, V):
        if t.stride(-1) != 1 or t.stride(-2) != dh:
            raise ValueError("K/V rows must be contiguous [H, dh]")
    if cu_offsets is None and (K.stride(0) != L_max * ks or V.stride(0) != L_max * vs):
        raise ValueError("dense K/V must have uniform row strides")
    P = P.contiguous()
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        if mask.dtype != torch.uint8 or mask.numel() != rows or mask.device != dev:
            raise ValueError(f"mask must be uint8/bool with {rows} elements on the same device")
        mask = mask.contiguous()
    pb = make_problem(B, H, m, dh, rows, L_max=L_max, dtype=dt, norm=norm, scale=scale or 0.0,
                      k_row_stride=ks, v_row_stride=vs, q_batch_stride=(H * m * dh if per_user else 0),
                      chunk_rows=chunk_rows, flags=SA_FLAG_CHECK_OFFSETS if check_offsets else 0)
    nws = sa_forward_workspace_size(pb)
    if nws == 0:
        _check(lib.sa_forward(ctypes.byref(pb), None, None, None, None, None, None, None, None, None, 0, None))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    S = out if out is not None else torch.empty((B, H, m, dh), dtype=torch.float32, device=dev)
    lse = None
    if return_lse:
        lse = torch.empty((B, H, m) if norm == "history" else (rows, H), dtype=torch.float32, device=dev)
    st = lib.sa_forward(ctypes.byref(pb), _ptr(P), _ptr(K), _ptr(V), _ptr(cu_offsets), _ptr(lengths), _ptr(mask),
                        _ptr(S), _ptr(lse), _ptr(workspace), nws, _stream_handle(dev))
    _check(st)
    return (S, lse) if return_lse else S


def sa_forward_fused_proj(X, Wk, Wv, P, cu_offsets, mask=None, norm: str = "history", return_lse: bool = False,
                          scale: float | None = None, chunk_rows: int = 0, workspace=None, out=None):
    """Fused K/V projection + Sketch Attention: K = X Wk, V = X Wv (V = X when
    ``Wv`` is None) computed on chip.  X [rows, d_model] bf16, Wk/Wv
    [d_model, H*dh], P [H, m, dh] (or [B, H, m, dh], per user), cu_offsets
    int32 [B+1]."""
    import torch
    lib = load_library()
    dev = X.device
    B = cu_offsets.numel() - 1
    per_user = P.dim() == 4
    if per_user and P.shape[0] != B:
        raise ValueError("per-user P must be [B, H, m, dh]")
    H, m, dh = P.shape[-3:]
    rows, d_model = X.shape
    for t in (X, Wk, P) + ((Wv,) if Wv is not None else ()):
        if t.device != dev or t.dtype != X.dtype:
            raise ValueError("X, Wk, Wv and P must share one device and dtype")
    X, Wk, P = X.contiguous(), Wk.contiguous(), P.contiguous()
    Wv = Wv.contiguous() if Wv is not None else None
    if mask is not None:
        mask = (mask.to(torch.uint8) if mask.dtype == torch.bool else mask).contiguous()
    pb = make_problem(B, H, m, dh, rows, dtype=_dtype_name(X), norm=norm, scale=scale or 0.0, chunk_rows=chunk_rows,
                      q_batch_stride=(H * m * dh if per_user else 0))
    nws = int(lib.sa_forward_fused_proj_workspace_size(ctypes.byref(pb), int(d_model)))
    if nws == 0:
        _check(lib.sa_forward_fused_proj(ctypes.byref(pb), None, int(d_model), None, None, None, None, None, None,
                                         None, None, 0, None))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    S = out if out is not None else torch.empty((B, H, m, dh), dtype=torch.float32, device=dev)
    lse = None
    if return_lse:
        lse = torch.empty((B, H, m) if norm == "history" else (rows, H), dtype=torch.float32, device=dev)
    st = lib.sa_forward_fused_proj(ctypes.byref(pb), _ptr(X), int(d_model), _ptr(Wk), _ptr(Wv), _ptr(P),
                                   _ptr(cu_offsets), _ptr(mask), _ptr(S), _ptr(lse), _ptr(workspace), nws,
                                   _stream_handle(dev))
    _check(st)
    return (S, lse) if return_lse else S


REFINE_KEYS = ("Wq", "Wk", "ln1_g", "ln1_b", "W1", "W3", "W2", "ln2_g", "ln2_b")


def sa_refine_forward(X, P0, layers, cu_offsets, H: int, mask=None, eps: float = 1e-5, scale: float | None = None,
                      workspace=None, out=None):
    """Stacked Sketch Attention refinement: ``len(layers)`` layers starting from
    the prototypes P0 [m, d] (fp32).  X [rows, d] bf16 (the history, also the
    values), cu_offsets int32 [B+1], H heads of d/H channels.  Each layer is a
    dict of device tensors: Wq, Wk [d, d], W1, W3 [d, 2d], W2 [2d, d] (bf16,
    [in, out]) and ln1_g, ln1_b, ln2_g, ln2_b [d] (fp32).  Returns the final
    sketch [B, m, d] fp32."""
    import torch
    lib = load_library()
    dev = X.device
    B = cu_offsets.numel() - 1
    rows, d = X.shape
    m = P0.shape[0]
    if P0.shape[1] != d or d % H:
        raise ValueError("P0 must be [m, d] with d a multiple of H")
    if X.dtype != torch.bfloat16 or P0.dtype != torch.float32:
        raise ValueError("X must be bf16 and P0 fp32")
    X, P0 = X.contiguous(), P0.contiguous()
    keep = []
    arr = (SaRefineLayer * len(layers))()
    for i, L in enumerate(layers):
        for k in REFINE_KEYS:
            t = L[k]
            want = torch.float32 if k.startswith("ln") else torch.bfloat16
            if t.device != dev or t.dtype != want:
                raise ValueError(f"layer {i}: {k} must be a {want} tensor on {dev}")
            t = t.contiguous()
            keep.append(t)
            setattr(arr[i], k, t.data_ptr())
    if mask is not None:
        mask = (mask.to(torch.uint8) if mask.dtype == torch.bool else mask).contiguous()
    pb = make_problem(B, H, m, d // H, rows, dtype="bf16", norm="history", scale=scale or 0.0)
    nl = len(layers)
    nws = int(lib.sa_refine_workspace_size(ctypes.byref(pb), int(d), nl))
    if nws == 0:
        _check(lib.sa_refine_forward(ctypes.byref(pb), None, int(d), None, nl, None, float(eps), None, None, None, None,
                                     0, None))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    out = out if out is not None else torch.empty((B, m, d), dtype=torch.float32, device=dev)
    st = lib.sa_refine_forward(ctypes.byref(pb), _ptr(X), int(d), _ptr(P0), nl, arr, float(eps), _ptr(cu_offsets),
                               _ptr(mask), _ptr(out), _ptr(workspace), nws, _stream_handle(dev))
    _check(st)
    return out


def sa_refine_workspace_size(pb, d_model: int, n_layers: int) -> int:
    return int(load_library().sa_refine_workspace_size(ctypes.byref(pb), int(d_model), int(n_layers)))


def sa_backward(P, K, V, S, lse, dS, cu_offsets=None, lengths=None, mask=None, scale: float | None = None,
                workspace=None, out=None, grad_dtype=None):
    """Gradients of the history-axis forward: returns (dP, dK, dV), dP in
    fp32 and dK, dV in ``grad_dtype`` (torch.float32, the default, or
    torch.bfloat16, the element type of K and V).  P, K, V, cu_offsets,
    lengths, mask as given to :func:`sa_forward`; S and lse its outputs; dS
    [B, H, m, dh] fp32.  dK and dV are zero-initialised here, so rows outside
    every user come back as 0."""
    import torch
    lib = load_library()
    dev = K.device
    packed = cu_offsets is not None
    H, m, dh = P.shape[-3:]
    if packed:
        B = cu_offsets.numel() - 1
        rows, L_max = K.shape[0], 0
    else:
        B, L_max = K.shape[0], K.shape[1]
        rows = B * L_max
    per_user = P.dim() == 4
    P, K, V = P.contiguous(), K.contiguous(), V.contiguous()
    S, lse, dS = S.contiguous(), lse.contiguous(), dS.to(torch.float32).contiguous()
    if mask is not None:
        mask = (mask.to(torch.uint8) if mask.dtype == torch.bool else mask).contiguous()
    if out is not None:
        grad_dtype = out[1].dtype
    grad_dtype = grad_dtype or torch.float32
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"grad_dtype must be torch.float32 or torch.bfloat16 (got {grad_dtype})")
    pb = make_problem(B, H, m, dh, rows, L_max=L_max, dtype=_dtype_name(K), scale=scale or 0.0,
                      q_batch_stride=(H * m * dh if per_user else 0),
                      flags=SA_FLAG_BF16_GRADS if grad_dtype == torch.bfloat16 else 0)
    nws = int(lib.sa_backward_workspace_size(ctypes.byref(pb)))
    if nws == 0:
        _check(lib.sa_backward(ctypes.byref(pb), *([None] * 13), 0, None))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    if out is None:
        dP = torch.empty(P.shape, dtype=torch.float32, device=dev)
        dK = torch.zeros(K.shape, dtype=grad_dtype, device=dev)
        dV = torch.zeros(V.shape, dtype=grad_dtype, device=dev)
    else:
        dP, dK, dV = out
        if dK.dtype != grad_dtype or dV.dtype != grad_dtype:
            raise ValueError("out: dK and dV must share one dtype")
    st = lib.sa_backward(ctypes.byref(pb), _ptr(P), _ptr(K), _ptr(V), _ptr(cu_offsets), _ptr(lengths), _ptr(mask),
                         _ptr(S), _ptr(lse), _ptr(dS), _ptr(dP), _ptr(dK), _ptr(dV), _ptr(workspace), nws,
                         _stream_handle(dev))
    _check(st)
    return dP, dK, dV


def sa_stca_attention(xt, X, Wq, Wk, Wv, cu_offsets, t_offsets, h: int, windows=None, scale: float | None = None,
                      workspace=None, out=None):
    """STCA single-query attention, reordered (appendix G.2.1), for every
    target: xt [T, D] and X [rows, D] bf16, Wq, Wk, Wv [D, D] bf16 ([in,
    out]), cu_offsets and t_offsets int32 [B+1] (user rows and user
    targets), windows int32 [T, 2] or None.  Returns out [T, D] fp32."""
    import torch
    lib = load_library()
    dev = xt.device
    T, D = xt.shape
    B = t_offsets.numel() - 1
    xt, Wq, Wk, Wv = (t.contiguous() for t in (xt, Wq, Wk, Wv))
    # X may be a row view of a wider buffer (unit column stride, rows apart)
    if X.dim() != 2 or X.stride(1) != 1 or X.stride(0) < D:
        X = X.contiguous()
    if windows is not None:
        windows = windows.to(torch.int32).contiguous()
    pb = SaStcaProblem(B=B, T=T, D=D, h=h, total_rows=X.shape[0], x_row_stride=X.stride(0), scale=scale or 0.0,
                       flags=0)
    nws = int(lib.sa_stca_workspace_size(ctypes.byref(pb)))
    if nws == 0:
        _check(lib.sa_stca_attention(ctypes.byref(pb), *([None] * 10), 0, None))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=dev)
    st = lib.sa_stca_attention(ctypes.byref(pb), _ptr(xt), _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(cu_offsets),
                               _ptr(t_offsets), _ptr(windows), _ptr(out), _ptr(workspace), nws, _stream_handle(dev))
    _check(st)
    return out


def sa_stca_workspace_size(pb) -> int:
    return int(load_library().sa_stca_workspace_size(ctypes.byref(pb)))


def sa_backward_workspace_size(pb) -> int:
    return int(load_library().sa_backward_workspace_size(ctypes.byref(pb)))
