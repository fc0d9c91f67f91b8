"""sa_forward_noalloc against sa_forward, through the C ABI: the same kernels
and plan over the library's own per-device workspace array instead of a
caller workspace, so the outputs must be bitwise equal.  Two calls in a row,
the second on a smaller input (the array keeps the first call's contents),
on the streaming kernels (both axes, and the pipelined dh = 128 one), the
register-staged kernel and the fp32 kernel; and a problem beyond the array is rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import device
import sketch_attention_flashsa_amd as sa

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(w, norm):
    """(S, lse) from sa_forward and from sa_forward_noalloc on the same inputs."""
    dev = device()
    P, K, V = (w[k].to(dev) for k in ("P", "K", "V"))
    packed = w["layout"] == "packed"
    cu = w["cu_offsets"].to(dev) if packed else None
    ln = None if packed else w["lengths"].to(dev)
    B, H, m, dh = w["B"], w["H"], w["m"], w["dh"]
    rows = K.shape[0] if packed else K.shape[0] * K.shape[1]
    S0, l0 = sa.sa_forward(P, K, V, cu_offsets=cu, lengths=ln, norm=norm, return_lse=True)
    pb = sa.make_problem(B, H, m, dh, rows, L_max=0 if packed else K.shape[1], dtype=w["dtype"], norm=norm)
    S1 = torch.full_like(S0, float("nan"))
    l1 = torch.full_like(l0, float("nan"))
    lib = sa.load_library()
    st = lib.sa_forward_noalloc(ctypes.byref(pb), _ptr(P), _ptr(K), _ptr(V), _ptr(cu), _ptr(ln), None, _ptr(S1),
                                _ptr(l1), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, sa.sa_last_error()
    torch.cuda.synchronize()
    return (S0, l0), (S1, l1)


@pytest.mark.parametrize("dtype,H,m,dh,norm,layout,big,small", [
    ("bf16", 8, 128, 64, "history", "packed", [30011, 1, 0, 20000, 4097], [700, 33]),
    ("bf16", 8, 128, 64, "prototype", "packed", [9000, 0, 2500], [64, 1, 31]),
    ("bf16", 3, 48, 32, "history", "dense", [4000, 17, 2100], [40, 0]),
    ("bf16", 1, 256, 128, "history", "packed", [5000, 1, 777], [40, 3]),
    ("f32", 2, 16, 32, "history", "packed", [3000, 1, 999], [5]),
])
def test_noalloc_equals_sa_forward_two_calls(dtype, H, m, dh, norm, layout, big, small):
    for i, lengths in enumerate((big, small)):
        w = W.random_case(700 + 10 * i + dh, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype=dtype,
                          layout=layout)
        (S0, l0), (S1, l1) = _both(w, norm)
        assert torch.equal(S0, S1), f"call {i + 1}: S differs from sa_forward"
        fin = torch.isfinite(l0)
        assert torch.equal(fin, torch.isfinite(l1)) and torch.equal(l0[fin], l1[fin]), f"call {i + 1}: lse differs"


def test_noalloc_rejects_problems_beyond_its_array():
    """2,000 users of the 100K workload's head shape need one partial-sum
    slot per user and row range, ~0.5 GB of workspace, more than the 64 MiB
    array: SA_ERR_WORKSPACE, outputs untouched."""
    dev = device()
    lib = sa.load_library()
    assert lib.sa_forward_noalloc_max_workspace() == 64 << 20
    pb = sa.make_problem(2000, 8, 128, 64, 1_600_000)
    assert sa.sa_forward_workspace_size(pb) > 64 << 20
    S = torch.full((2000, 8, 128, 64), 3.0, dtype=torch.float32, device=dev)
    fake = ctypes.c_void_p(1 << 20)      # never used: the call fails on the host first
    st = lib.sa_forward_noalloc(ctypes.byref(pb), fake, fake, fake, fake, None, None, _ptr(S), None,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == sa.SA_ERR_WORKSPACE and "workspace" in sa.sa_last_error()
    torch.cuda.synchronize()
    assert torch.all(S == 3.0)
