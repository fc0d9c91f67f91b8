"""GPU checks of the C ABI's contracts beyond the numbers: the debug offsets
check (SA_FLAG_CHECK_OFFSETS), that a call writes nothing outside its
outputs and workspace (guard bytes on both sides of every output and of the
workspace), and that the timing events are forgotten by a call that fails.

The offsets check is exercised only with offsets whose rows all lie inside
the K/V buffers (decreasing pairs): even an unchecked kernel would stay in
bounds there.  The other rules are covered on the host
(tests/test_abi.py), where the same rule code runs."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_lse, assert_parity, device, run
import sketch_attention_flashsa_amd as sa

pytestmark = pytest.mark.gpu

GUARD = 256
PATTERN = 0xA5


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Guarded:
    """A device region of `nbytes` with GUARD bytes of a fixed pattern before
    and after it (the region itself starts 256-byte aligned)."""

    def __init__(self, nbytes, dev):
        self.nbytes = int(nbytes)
        body = (self.nbytes + 255) // 256 * 256
        self.buf = torch.full((GUARD + body + GUARD,), PATTERN, dtype=torch.uint8, device=dev)
        self.ptr = ctypes.c_void_p(self.buf.data_ptr() + GUARD)

    def view(self, dtype, shape):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.buf[GUARD:GUARD + n].view(dtype).view(shape)

    def assert_intact(self, what):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        head, tail = b[:GUARD], b[GUARD + self.nbytes:]
        assert np.all(head == PATTERN), f"{what}: bytes before the region were written"
        assert np.all(tail == PATTERN), f"{what}: bytes after the region were written"


def _forward_raw(pb, P, K, V, cu, lengths, mask, S, lse, ws, nws):
    lib = sa.load_library()
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.sa_forward(ctypes.byref(pb), ptr(P), ptr(K), ptr(V), ptr(cu), ptr(lengths), ptr(mask),
                          S if isinstance(S, ctypes.c_void_p) else ptr(S),
                          lse if isinstance(lse, ctypes.c_void_p) or lse is None else ptr(lse),
                          ws if isinstance(ws, ctypes.c_void_p) else ptr(ws), nws, _stream())


# ------------------------------------------------------------ offsets check
@pytest.mark.parametrize("norm", ["history", "prototype"])
def test_check_offsets_valid_offsets_change_nothing(norm):
    """With valid offsets the check reports status 0 (first bad -1) and the
    results equal the unchecked call bitwise."""
    dev = device()
    w = W.random_case(301, B=5, H=8, m=128, dh=64, lengths=[900, 0, 1, 2049, 77], dtype="bf16")
    P, K, V, cu = (w[k].to(dev) for k in ("P", "K", "V", "cu_offsets"))
    S0, l0 = sa.sa_forward(P, K, V, cu_offsets=cu, norm=norm, return_lse=True)
    pb = sa.make_problem(5, 8, 128, 64, K.shape[0], norm=norm, flags=sa.SA_FLAG_CHECK_OFFSETS)
    ws = torch.empty(sa.sa_forward_workspace_size(pb), dtype=torch.uint8, device=dev)
    S1, l1 = sa.sa_forward(P, K, V, cu_offsets=cu, norm=norm, return_lse=True, workspace=ws, check_offsets=True)
    torch.cuda.synchronize()
    status = ws[:8].view(torch.int32).cpu().tolist()
    assert status == [0, -1], status
    assert torch.equal(S0, S1) and torch.equal(l0, l1)


@pytest.mark.parametrize("norm", ["history", "prototype"])
def test_check_offsets_rejects_decreasing_offsets(norm):
    """A decreasing pair (rows still inside the buffer): status 2 with the
    first bad index, S and lse all NaN, the call itself returns OK."""
    dev = device()
    w = W.random_case(302, B=3, H=2, m=64, dh=32, lengths=[500, 300, 200], dtype="bf16")
    P, K, V = (w[k].to(dev) for k in ("P", "K", "V"))
    cu = torch.tensor([0, 500, 300, 1000], dtype=torch.int32, device=dev)
    bits, first = sa.sa_check_offsets_host(cu.cpu().numpy(), K.shape[0])
    assert (bits, first) == (2, 1)
    pb = sa.make_problem(3, 2, 64, 32, K.shape[0], norm=norm, flags=sa.SA_FLAG_CHECK_OFFSETS)
    ws = torch.empty(sa.sa_forward_workspace_size(pb), dtype=torch.uint8, device=dev)
    S, lse = sa.sa_forward(P, K, V, cu_offsets=cu, norm=norm, return_lse=True, workspace=ws, check_offsets=True)
    torch.cuda.synchronize()
    assert ws[:8].view(torch.int32).cpu().tolist() == [2, 1]
    assert torch.isnan(S).all() and torch.isnan(lse).all()
    # the same workspace serves a valid call next: the status is rewritten
    cu_ok = torch.tensor([0, 300, 500, 1000], dtype=torch.int32, device=dev)
    S2 = sa.sa_forward(P, K, V, cu_offsets=cu_ok, norm=norm, workspace=ws, check_offsets=True)
    torch.cuda.synchronize()
    assert ws[:8].view(torch.int32).cpu().tolist() == [0, -1]
    So, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=cu_ok.cpu(), norm=norm)
    assert_parity(S2.double().cpu().numpy(), So, "bf16", f"checked call after a rejected one ({norm})")


def test_check_offsets_fused_entry():
    """The fused projection entry runs the same check (decreasing pair inside
    the buffer): status 2, S NaN; valid offsets give status 0 and the
    unchecked result."""
    dev = device()
    w = W.random_fused_case(303, B=3, H=8, m=64, dh=32, d_model=256, lengths=[400, 100, 700])
    X, Wk, Wv, P = (w[k].to(dev) for k in ("X", "Wk", "Wv", "P"))
    cu_ok = w["cu_offsets"].to(dev)
    pb = sa.make_problem(3, 8, 64, 32, X.shape[0], flags=sa.SA_FLAG_CHECK_OFFSETS)
    nws = int(sa.load_library().sa_forward_fused_proj_workspace_size(ctypes.byref(pb), 256))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    lib = sa.load_library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    for cu, want in ((cu_ok, [0, -1]), (torch.tensor([0, 400, 100, 1200], dtype=torch.int32, device=dev), [2, 1])):
        S = torch.empty((3, 8, 64, 32), dtype=torch.float32, device=dev)
        st = lib.sa_forward_fused_proj(ctypes.byref(pb), ptr(X), 256, ptr(Wk), ptr(Wv), ptr(P), ptr(cu), None, ptr(S),
                                       None, ptr(ws), nws, _stream())
        assert st == 0, sa.sa_last_error()
        torch.cuda.synchronize()
        assert ws[:8].view(torch.int32).cpu().tolist() == want
        if want[0]:
            assert torch.isnan(S).all()
        else:
            S0 = sa.sa_forward_fused_proj(X, Wk, Wv, P, cu)
            assert torch.equal(S, S0)


def test_check_offsets_dense_layout_has_nothing_to_check():
    dev = device()
    w = W.random_case(304, B=3, H=2, m=32, dh=32, lengths=[40, 0, 90], dtype="bf16", layout="dense")
    P, K, V, ln = (w[k].to(dev) for k in ("P", "K", "V", "lengths"))
    S0 = sa.sa_forward(P, K, V, lengths=ln)
    pb = sa.make_problem(3, 2, 32, 32, K.shape[0] * K.shape[1], L_max=K.shape[1], flags=sa.SA_FLAG_CHECK_OFFSETS)
    ws = torch.full((sa.sa_forward_workspace_size(pb),), 7, dtype=torch.uint8, device=dev)
    S1 = sa.sa_forward(P, K, V, lengths=ln, workspace=ws, check_offsets=True)
    torch.cuda.synchronize()
    assert ws[:8].view(torch.int32).cpu().tolist() == [0, -1]
    assert torch.equal(S0, S1)


# ----------------------------------------------------------- guard canaries
@pytest.mark.parametrize("dtype,H,m,dh,norm,layout", [
    ("bf16", 8, 128, 64, "history", "packed"),
    ("bf16", 8, 128, 64, "prototype", "packed"),
    ("bf16", 3, 48, 32, "history", "dense"),
    ("bf16", 1, 256, 128, "history", "packed"),
    ("f32", 2, 16, 32, "history", "packed"),
])
def test_forward_writes_only_its_outputs(dtype, H, m, dh, norm, layout):
    """S, lse and the workspace each sit between guard bytes; after a normal
    call the guards are untouched and S matches the oracle."""
    dev = device()
    lengths = [700, 0, 33, 1500, 1]
    w = W.random_case(310 + dh + H, B=5, H=H, m=m, dh=dh, lengths=lengths, dtype=dtype, layout=layout)
    P, K, V = (w[k].to(dev) for k in ("P", "K", "V"))
    cu = w["cu_offsets"].to(dev) if layout == "packed" else None
    ln = w["lengths"].to(dev) if layout == "dense" else None
    rows = K.shape[0] if layout == "packed" else K.shape[0] * K.shape[1]
    pb = sa.make_problem(5, H, m, dh, rows, L_max=0 if layout == "packed" else K.shape[1], dtype=dtype, norm=norm,
                         k_row_stride=H * dh, v_row_stride=H * dh)
    nws = sa.sa_forward_workspace_size(pb)
    nS = 5 * H * m * dh * 4
    nl = (5 * H * m if norm == "history" else rows * H) * 4
    gS, gl, gw = Guarded(nS, dev), Guarded(nl, dev), Guarded(max(nws, 1), dev)
    st = _forward_raw(pb, P, K, V, cu, ln, None, gS.ptr, gl.ptr, gw.ptr, nws)
    assert st == 0, sa.sa_last_error()
    for g, what in ((gS, "S"), (gl, "lse"), (gw, "workspace")):
        g.assert_intact(f"{what} ({dtype} H={H} m={m} dh={dh} {norm} {layout})")
    S = gS.view(torch.float32, (5, H, m, dh)).double().cpu().numpy()
    if layout == "packed":
        So, _ = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], norm=norm)
    else:
        So, _ = oracle.forward(w["P"], w["K"], w["V"], lengths=w["lengths"], norm=norm)
    assert_parity(S, So, dtype, "guarded call")


def test_backward_writes_only_its_outputs():
    """dP, dK, dV and the workspace between guard bytes (dK and dV are
    written for every row of a user, never past the buffer)."""
    dev = device()
    w = W.random_case(320, B=3, H=8, m=128, dh=64, lengths=[600, 1, 900], dtype="bf16")
    P, K, V, cu = (w[k].to(dev) for k in ("P", "K", "V", "cu_offsets"))
    S, lse = sa.sa_forward(P, K, V, cu_offsets=cu, return_lse=True)
    dS = torch.from_numpy(np.random.default_rng(5).standard_normal(S.shape, dtype=np.float32)).to(dev)
    rows = K.shape[0]
    pb = sa.make_problem(3, 8, 128, 64, rows)
    nws = sa.sa_backward_workspace_size(pb)
    gP, gK, gV, gw = (Guarded(P.numel() * 4, dev), Guarded(rows * 8 * 64 * 4, dev), Guarded(rows * 8 * 64 * 4, dev),
                      Guarded(nws, dev))
    lib = sa.load_library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.sa_backward(ctypes.byref(pb), ptr(P), ptr(K), ptr(V), ptr(cu), None, None, ptr(S), ptr(lse), ptr(dS),
                         gP.ptr, gK.ptr, gV.ptr, gw.ptr, nws, _stream())
    assert st == 0, sa.sa_last_error()
    for g, what in ((gP, "dP"), (gK, "dK"), (gV, "dV"), (gw, "workspace")):
        g.assert_intact(f"backward {what}")
    dP_ref, dK_ref, dV_ref = sa.sa_backward(P, K, V, S, lse, dS, cu_offsets=cu)
    assert torch.equal(gP.view(torch.float32, tuple(P.shape)), dP_ref)
    assert torch.equal(gK.view(torch.float32, tuple(K.shape)), dK_ref)
    assert torch.equal(gV.view(torch.float32, tuple(V.shape)), dV_ref)


def test_fused_writes_only_its_outputs():
    dev = device()
    w = W.random_fused_case(330, B=3, H=8, m=256, dh=32, d_model=256, lengths=[1000, 1, 2000])
    X, Wk, Wv, P, cu = (w[k].to(dev) for k in ("X", "Wk", "Wv", "P", "cu_offsets"))
    pb = sa.make_problem(3, 8, 256, 32, X.shape[0])
    lib = sa.load_library()
    nws = int(lib.sa_forward_fused_proj_workspace_size(ctypes.byref(pb), 256))
    gS, gl, gw = Guarded(3 * 8 * 256 * 32 * 4, dev), Guarded(3 * 8 * 256 * 4, dev), Guarded(nws, dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.sa_forward_fused_proj(ctypes.byref(pb), ptr(X), 256, ptr(Wk), ptr(Wv), ptr(P), ptr(cu), None, gS.ptr,
                                   gl.ptr, gw.ptr, nws, _stream())
    assert st == 0, sa.sa_last_error()
    for g, what in ((gS, "S"), (gl, "lse"), (gw, "workspace")):
        g.assert_intact(f"fused {what}")
    S_ref = sa.sa_forward_fused_proj(X, Wk, Wv, P, cu)
    assert torch.equal(gS.view(torch.float32, (3, 8, 256, 32)), S_ref)


# ------------------------------------------------------------ timing events
def test_timing_events_forgotten_by_a_failing_call():
    """Events armed before a call that fails validation are not recorded by
    the next successful call; armed before a successful call they are."""
    dev = device()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipGetLastError.restype = ctypes.c_int
    evs = [ctypes.c_void_p() for _ in range(4)]
    for e in evs:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    w = W.random_case(340, B=2, H=2, m=32, dh=32, lengths=[300, 200], dtype="bf16")
    P, K, V, cu = (w[k].to(dev) for k in ("P", "K", "V", "cu_offsets"))
    try:
        sa.sa_set_timing_events(evs[0], evs[1])
        bad = sa.make_problem(-1, 2, 32, 32, K.shape[0])
        assert _forward_raw(bad, P, K, V, cu, None, None, ctypes.c_void_p(0), None, ctypes.c_void_p(0), 0) != 0
        sa.sa_forward(P, K, V, cu_offsets=cu)
        sa.sa_set_timing_events(evs[2], evs[3])
        sa.sa_forward(P, K, V, cu_offsets=cu)
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[2], evs[3]) == 0 and ms.value >= 0.0
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) != 0, \
            "events armed before a failing call must not be recorded by a later call"
        # that query's error is left pending in the runtime: the next call
        # must still report only its own launches
        S = sa.sa_forward(P, K, V, cu_offsets=cu)
        torch.cuda.synchronize()
        assert torch.isfinite(S).all()
    finally:
        hip.hipGetLastError()
        sa.sa_set_timing_events(None, None)
        for e in evs:
            hip.hipEventDestroy(e)
