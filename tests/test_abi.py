"""The C ABI without a GPU: the library loads, exports every function the
header declares, the Python mirror of sa_problem matches the header, and
host-detectable errors return a status before anything is enqueued."""
import ctypes
import os
import re

import pytest

import sketch_attention_flashsa_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sketchattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sa.LIB_PATH), reason="libsketchattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(sa_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) == set(sa.EXPORTED), names
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_problem_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct sa_problem \{(.*?)\} sa_problem;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int32_t|int64_t|float)\s+([\w, ]+);", body)
    names = [n.strip() for _, group in fields for n in group.split(",")]
    assert names == [f[0] for f in sa.SaProblem._fields_]
    ctypes_of = {"int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "float": ctypes.c_float}
    types = [ctypes_of[t] for t, group in fields for _ in group.split(",")]
    assert types == [f[1] for f in sa.SaProblem._fields_]


def test_version_and_status_strings():
    assert sa.sa_version() == 100
    assert sa.sa_status_string(0) == "ok"
    assert "workspace" in sa.sa_status_string(3)
    assert sa.sa_status_string(99) == "unknown status"


def _call(pb, **ptrs):
    lib = sa.load_library()
    p = {k: ptrs.get(k) for k in ("P", "K", "V", "cu", "len", "mask", "S", "lse", "ws")}
    return lib.sa_forward(ctypes.byref(pb), p["P"], p["K"], p["V"], p["cu"], p["len"], p["mask"], p["S"], p["lse"],
                          p["ws"], ptrs.get("nws", 0), None)


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("field,value,status", [
    ("B", -1, sa.SA_ERR_INVALID_ARG),
    ("H", 0, sa.SA_ERR_INVALID_ARG),
    ("dtype", 7, sa.SA_ERR_INVALID_ARG),
    ("norm", 5, sa.SA_ERR_INVALID_ARG),
    ("flags", 1, sa.SA_ERR_INVALID_ARG),
    ("flags", 4, sa.SA_ERR_INVALID_ARG),
    ("chunk_rows", 33, sa.SA_ERR_INVALID_ARG),
    ("dh", 48, sa.SA_ERR_UNSUPPORTED),
    ("m", 40, sa.SA_ERR_UNSUPPORTED),
    ("k_row_stride", 7, sa.SA_ERR_INVALID_ARG),
    ("total_rows", -5, sa.SA_ERR_INVALID_ARG),
])
def test_invalid_problem_rejected(field, value, status):
    pb = sa.make_problem(2, 4, 64, 32, 100, dtype="bf16")
    setattr(pb, field, value)
    st = _call(pb, P=FAKE, K=FAKE, V=FAKE, cu=FAKE, S=FAKE)
    assert st == status, (st, sa.sa_last_error())
    assert sa.sa_last_error() != ""


def test_null_pointers_and_workspace_rejected():
    pb = sa.make_problem(2, 4, 64, 32, 100, dtype="bf16")
    assert _call(pb, P=None, K=FAKE, V=FAKE, cu=FAKE, S=FAKE) == sa.SA_ERR_INVALID_ARG
    nws = sa.sa_forward_workspace_size(pb)
    assert nws > 0
    assert _call(pb, P=FAKE, K=FAKE, V=FAKE, cu=FAKE, S=FAKE, ws=None, nws=0) == sa.SA_ERR_WORKSPACE
    assert _call(pb, P=FAKE, K=FAKE, V=FAKE, cu=FAKE, S=FAKE, ws=FAKE, nws=nws - 1) == sa.SA_ERR_WORKSPACE
    # packed layout must not carry L_max
    pb2 = sa.make_problem(2, 4, 64, 32, 100, L_max=10, dtype="bf16")
    assert _call(pb2, P=FAKE, K=FAKE, V=FAKE, cu=FAKE, S=FAKE) == sa.SA_ERR_INVALID_ARG
    # misaligned bf16 pointer
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert _call(pb, P=FAKE, K=odd, V=FAKE, cu=FAKE, S=FAKE, ws=FAKE, nws=nws) == sa.SA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op():
    pb = sa.make_problem(0, 4, 64, 32, 0, dtype="bf16")
    assert _call(pb, cu=FAKE) == sa.SA_OK


def test_workspace_size_is_layout_independent_and_monotone():
    a = sa.sa_forward_workspace_size(sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16"))
    b = sa.sa_forward_workspace_size(sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16", norm="prototype"))
    # the one-pass prototype axis keeps no per-row state between passes
    assert 0 < a == b
    # a two-pass shape (m not a multiple of 32) adds the per-row normaliser
    c = sa.sa_forward_workspace_size(sa.make_problem(16, 8, 48, 64, 1_600_000, dtype="bf16"))
    d = sa.sa_forward_workspace_size(sa.make_problem(16, 8, 48, 64, 1_600_000, dtype="bf16", norm="prototype"))
    assert d == c + ((1_600_000 * 8 * 4 + 255) // 256) * 256
    # partials stay a small fraction of the K/V bytes at the 100K workload
    assert a < 0.05 * (2 * 1_600_000 * 8 * 64 * 2)


def test_kernel_name_query():
    # the streaming kernel serves the 64- and 32-wide heads; f32 has its own kernel
    assert sa.sa_forward_kernel_name(sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16")) == "sa_bf16_stream_kernel"
    assert sa.sa_forward_kernel_name(sa.make_problem(8, 4, 64, 32, 4096, dtype="bf16")) == "sa_bf16_stream_kernel"
    # their prototype axis runs in one pass
    assert sa.sa_forward_kernel_name(sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16", norm="prototype")) == \
        "sa_proto_stream_kernel"
    assert sa.sa_forward_kernel_name(sa.make_problem(8, 4, 64, 32, 4096, dtype="bf16", norm="prototype")) == \
        "sa_proto_stream_kernel"
    assert sa.sa_forward_kernel_name(sa.make_problem(8, 2, 16, 16, 4096, dtype="f32")) == "sa_f32_fwd_kernel"
    # dh = 128 is outside the streaming kernel's shapes and uses the tiled kernel
    assert sa.sa_forward_kernel_name(sa.make_problem(8, 2, 64, 128, 4096, dtype="bf16")) == "sa_bf16_fwd_kernel"
    with pytest.raises(sa.SketchAttnError):
        sa.sa_forward_kernel_name(sa.make_problem(8, 0, 64, 32, 4096, dtype="bf16"))


def test_fused_entry_validation():
    lib = sa.load_library()
    pb = sa.make_problem(128, 8, 256, 32, 4_240_293, dtype="bf16")
    n = lib.sa_forward_fused_proj_workspace_size(ctypes.byref(pb), 256)
    assert n > 0
    # unsupported: d_model outside {128, 256}, dh != 32, fp32 inputs, prototype axis
    for bad, dm in ((sa.make_problem(4, 8, 256, 32, 1000, dtype="bf16"), 192),
                    (sa.make_problem(4, 8, 128, 64, 1000, dtype="bf16"), 256),
                    (sa.make_problem(4, 8, 128, 32, 1000, dtype="f32"), 256),
                    (sa.make_problem(4, 8, 128, 32, 1000, dtype="bf16", norm="prototype"), 256)):
        assert lib.sa_forward_fused_proj_workspace_size(ctypes.byref(bad), dm) == 0
        st = lib.sa_forward_fused_proj(ctypes.byref(bad), None, dm, None, None, None, None, None, None, None, None,
                                       0, None)
        assert st == sa.SA_ERR_UNSUPPORTED, sa.sa_last_error()
    # packed only, and V = X needs H*dh == d_model: rejected before any GPU work
    st = lib.sa_forward_fused_proj(ctypes.byref(pb), FAKE, 256, FAKE, None, FAKE, None, None, FAKE, None, FAKE,
                                   n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "cu_offsets" in sa.sa_last_error()
    pb5 = sa.make_problem(4, 5, 64, 32, 1000, dtype="bf16")
    n5 = lib.sa_forward_fused_proj_workspace_size(ctypes.byref(pb5), 256)
    st = lib.sa_forward_fused_proj(ctypes.byref(pb5), FAKE, 256, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE,
                                   n5, None)
    assert st == sa.SA_ERR_INVALID_ARG and "H*dh == d_model" in sa.sa_last_error()


def test_refine_entry_validation():
    lib = sa.load_library()
    pb = sa.make_problem(128, 8, 256, 32, 4_240_293, dtype="bf16")
    n = lib.sa_refine_workspace_size(ctypes.byref(pb), 256, 2)
    n1 = lib.sa_refine_workspace_size(ctypes.byref(pb), 256, 1)
    # the attention workspace plus xhat, queries and 7 d^2 bf16 weights per layer
    assert n > n1 > lib.sa_forward_fused_proj_workspace_size(ctypes.byref(pb), 256)
    assert n - n1 == 7 * 256 * 256 * 2
    # H*dh != d_model, n_layers out of range, fp32 inputs, dh != 32, d_model 192
    bad = [(sa.make_problem(4, 4, 256, 32, 1000, dtype="bf16"), 256, 2, sa.SA_ERR_INVALID_ARG),
           (pb, 256, 0, sa.SA_ERR_INVALID_ARG), (pb, 256, 9, sa.SA_ERR_INVALID_ARG),
           (sa.make_problem(4, 8, 128, 32, 1000, dtype="f32"), 256, 2, sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(4, 4, 128, 64, 1000, dtype="bf16"), 256, 2, sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(4, 6, 128, 32, 1000, dtype="bf16"), 192, 2, sa.SA_ERR_UNSUPPORTED)]
    for p, dm, nl, code in bad:
        assert lib.sa_refine_workspace_size(ctypes.byref(p), dm, nl) == 0
        st = lib.sa_refine_forward(ctypes.byref(p), None, dm, None, nl, None, 1e-5, None, None, None, None, 0, None)
        assert st == code, (st, sa.sa_last_error())
    # packed only, layers required, eps checked: all before any GPU work
    layers = (sa.SaRefineLayer * 2)()
    st = lib.sa_refine_forward(ctypes.byref(pb), FAKE, 256, FAKE, 2, layers, 1e-5, None, None, FAKE, FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "cu_offsets" in sa.sa_last_error()
    st = lib.sa_refine_forward(ctypes.byref(pb), FAKE, 256, FAKE, 2, None, 1e-5, FAKE, None, FAKE, FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "layers" in sa.sa_last_error()
    st = lib.sa_refine_forward(ctypes.byref(pb), FAKE, 256, FAKE, 2, layers, float("nan"), FAKE, None, FAKE, FAKE, n,
                               None)
    assert st == sa.SA_ERR_INVALID_ARG and "eps" in sa.sa_last_error()
    st = lib.sa_refine_forward(ctypes.byref(pb), FAKE, 256, FAKE, 2, layers, 1e-5, FAKE, None, FAKE, FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "non-NULL" in sa.sa_last_error()
    pq = sa.make_problem(4, 8, 256, 32, 1000, dtype="bf16", q_batch_stride=8 * 256 * 32)
    assert lib.sa_refine_workspace_size(ctypes.byref(pq), 256, 2) == 0


def test_backward_entry_validation():
    lib = sa.load_library()
    pb = sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16")
    n = lib.sa_backward_workspace_size(ctypes.byref(pb))
    assert n > 0
    bad = [(sa.make_problem(4, 8, 128, 64, 1000, dtype="f32"), sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(4, 8, 128, 64, 1000, dtype="bf16", norm="prototype"), sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(4, 8, 128, 128, 1000, dtype="bf16"), sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(4, 8, 48, 32, 1000, dtype="bf16"), sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(4, 8, 512, 32, 1000, dtype="bf16"), sa.SA_ERR_UNSUPPORTED),
           (sa.make_problem(-1, 8, 128, 64, 1000, dtype="bf16"), sa.SA_ERR_INVALID_ARG)]
    for p, code in bad:
        assert lib.sa_backward_workspace_size(ctypes.byref(p)) == 0
        st = lib.sa_backward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 1 << 30, None)
        assert st == code, (st, sa.sa_last_error())
    # required pointers, workspace size: rejected before any GPU work
    st = lib.sa_backward(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                         FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "non-NULL" in sa.sa_last_error()
    st = lib.sa_backward(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, n - 1, None)
    assert st == sa.SA_ERR_WORKSPACE
    st = lib.sa_backward(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "lengths" in sa.sa_last_error()
    # dK and dV take 16-byte vector stores
    odd = ctypes.c_void_p((1 << 20) + 4)
    st = lib.sa_backward(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, odd, FAKE,
                         FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "aligned" in sa.sa_last_error()


def test_bf16_gradient_flag():
    """SA_FLAG_BF16_GRADS is a backward-only flag: accepted there with the
    same workspace, rejected by the forward; other bits are rejected."""
    lib = sa.load_library()
    pb = sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16")
    pf = sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16", flags=sa.SA_FLAG_BF16_GRADS)
    n = lib.sa_backward_workspace_size(ctypes.byref(pb))
    assert n > 0 and lib.sa_backward_workspace_size(ctypes.byref(pf)) == n
    st = lib.sa_backward(ctypes.byref(pf), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, n - 1, None)
    assert st == sa.SA_ERR_WORKSPACE, sa.sa_last_error()
    bad = sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16", flags=2)
    assert lib.sa_backward_workspace_size(ctypes.byref(bad)) == 0
    st = lib.sa_backward(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "flags" in sa.sa_last_error()
    assert sa.sa_forward_workspace_size(pf) == 0
    assert _call(pf, P=FAKE, K=FAKE, V=FAKE, cu=FAKE, S=FAKE) == sa.SA_ERR_INVALID_ARG


def test_fused_two_pass_shapes():
    """Single head of width 128 with 1024 prototypes (the paper's production
    shape) folds W_K into the prototypes: its workspace is the streaming
    forward's plus the folded prototypes, no K; accepted with V = X, rejected
    with Wv.  Two heads of width 128 over d_model = 256 project K into the
    workspace instead."""
    lib = sa.load_library()
    pb = sa.make_problem(16, 1, 1024, 128, 1_600_000, dtype="bf16")
    n = lib.sa_forward_fused_proj_workspace_size(ctypes.byref(pb), 128)
    assert n == lib.sa_forward_workspace_size(ctypes.byref(pb)) + 1024 * 128 * 2
    st = lib.sa_forward_fused_proj(ctypes.byref(pb), FAKE, 128, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, n, None)
    assert st == sa.SA_ERR_UNSUPPORTED and "V = X only" in sa.sa_last_error()
    p2 = sa.make_problem(16, 2, 256, 128, 1_600_000, dtype="bf16")
    n2 = lib.sa_forward_fused_proj_workspace_size(ctypes.byref(p2), 256)
    # the streaming forward's workspace plus K (bf16, rows x 256) and W^T
    assert n2 >= lib.sa_forward_workspace_size(ctypes.byref(p2)) + 1_600_000 * 256 * 2 + 256 * 256 * 2
    # per-user P, H*dh != d_model, or a shape the streaming kernel does not take: unsupported
    for p, dm in ((sa.make_problem(4, 1, 1024, 128, 1000, dtype="bf16", q_batch_stride=1024 * 128), 128),
                  (sa.make_problem(4, 1, 1024, 128, 1000, dtype="bf16"), 256),
                  (sa.make_problem(4, 1, 1000, 128, 1000, dtype="bf16"), 128)):
        assert lib.sa_forward_fused_proj_workspace_size(ctypes.byref(p), dm) == 0
    # refinement keeps to the on-chip shapes
    assert lib.sa_refine_workspace_size(ctypes.byref(sa.make_problem(4, 1, 1024, 128, 1000, dtype="bf16")), 128, 2) == 0


def test_stca_entry_validation():
    lib = sa.load_library()

    def P(B=64, T=2560, D=1024, h=16, rows=65536, stride=0, scale=0.0, flags=0):
        return sa.SaStcaProblem(B=B, T=T, D=D, h=h, total_rows=rows, x_row_stride=stride, scale=scale, flags=flags)

    pb = P()
    n = lib.sa_stca_workspace_size(ctypes.byref(pb))
    # W_Q^T and W_V^T (bf16), a 32-byte block-table entry per block, the
    # queries [T, D] and alpha X [T, h, D] (bf16)
    grid = ((2560 // 16 + 64) * 8 + 7) // 8 * 8
    assert n >= 2 * 1024 * 1024 * 2 + 32 * grid + 2 * 2560 * 1024 + 2 * 2560 * 16 * 1024
    bad = [(P(D=512, h=8), sa.SA_ERR_UNSUPPORTED), (P(h=32), sa.SA_ERR_UNSUPPORTED),
           (P(h=15), sa.SA_ERR_INVALID_ARG), (P(B=-1), sa.SA_ERR_INVALID_ARG), (P(T=-3), sa.SA_ERR_INVALID_ARG),
           (P(stride=1000), sa.SA_ERR_INVALID_ARG), (P(stride=1028), sa.SA_ERR_INVALID_ARG),
           (P(scale=float("nan")), sa.SA_ERR_INVALID_ARG), (P(flags=1), sa.SA_ERR_INVALID_ARG)]
    for p, code in bad:
        assert lib.sa_stca_workspace_size(ctypes.byref(p)) == 0
        st = lib.sa_stca_attention(ctypes.byref(p), *([FAKE] * 10), 1 << 30, None)
        assert st == code, (st, sa.sa_last_error())
    assert lib.sa_stca_workspace_size(ctypes.byref(P(h=8))) > 0            # dh = 128
    assert lib.sa_stca_workspace_size(ctypes.byref(P(stride=2048))) > 0    # rows 2048 elements apart
    # required pointers and workspace: rejected before any GPU work; T == 0 is a no-op
    st = lib.sa_stca_attention(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, n, None)
    assert st == sa.SA_ERR_INVALID_ARG and "t_offsets" in sa.sa_last_error()
    st = lib.sa_stca_attention(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, n - 1,
                               None)
    assert st == sa.SA_ERR_WORKSPACE
    assert lib.sa_stca_attention(ctypes.byref(P(T=0)), *([None] * 10), 0, None) == sa.SA_OK


def test_stca_problem_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct sa_stca_problem \{(.*?)\} sa_stca_problem;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int32_t|int64_t|float)\s+([\w, ]+);", body)
    assert [n.strip() for _, grp in fields for n in grp.split(",")] == [f[0] for f in sa.SaStcaProblem._fields_]
    ctypes_of = {"int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "float": ctypes.c_float}
    assert [ctypes_of[t] for t, grp in fields for _ in grp.split(",")] == [f[1] for f in sa.SaStcaProblem._fields_]


def test_tuning_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct sa_tuning \{(.*?)\} sa_tuning;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"int32_t\s+(\w+);", body)
    assert names == [f[0] for f in sa.SaTuning._fields_]


def test_tuning_is_explicit_validated_and_thread_local():
    """The work split follows sa_set_tuning() only (never the environment):
    blocks per CU change the row ranges and so the workspace; invalid values
    are rejected without changing the settings; NULL restores the defaults;
    another thread keeps its own (default) settings."""
    import threading
    pb = sa.make_problem(16, 8, 128, 64, 1_600_000, dtype="bf16")
    base = sa.sa_forward_workspace_size(pb)
    os.environ["SA_BLOCKS_PER_CU"] = "8"      # must have no effect
    try:
        assert sa.sa_forward_workspace_size(pb) == base
    finally:
        del os.environ["SA_BLOCKS_PER_CU"]
    try:
        sa.sa_set_tuning(blocks_per_cu=8)
        tuned = sa.sa_forward_workspace_size(pb)
        assert tuned > base
        other = []
        t = threading.Thread(target=lambda: other.append(sa.sa_forward_workspace_size(pb)))
        t.start()
        t.join()
        assert other == [base], "tuning must be per thread"
        for bad in ({"stream_waves": 12}, {"range_split": 100}, {"blocks_per_cu": -1}, {"bf16_tile_mb": 32},
                    {"bf16_tile_mb": 24, "bf16_tile_nw": 4}, {"register_staged": 2}):
            with pytest.raises(sa.SketchAttnError):
                sa.sa_set_tuning(**bad)
            assert sa.sa_forward_workspace_size(pb) == tuned
        sa.sa_set_tuning(register_staged=1)
        assert sa.sa_forward_kernel_name(pb) == "sa_bf16_fwd_kernel"
    finally:
        sa.sa_set_tuning()
    assert sa.sa_forward_workspace_size(pb) == base
    assert sa.sa_forward_kernel_name(pb) == "sa_bf16_stream_kernel"


def test_check_offsets_flag_accepted_where_documented():
    """SA_FLAG_CHECK_OFFSETS: the forward entries accept it and need 256 bytes
    more workspace; refinement and the backward pass reject it."""
    pb = sa.make_problem(4, 8, 128, 64, 10_000, dtype="bf16")
    pc = sa.make_problem(4, 8, 128, 64, 10_000, dtype="bf16", flags=sa.SA_FLAG_CHECK_OFFSETS)
    assert sa.sa_forward_workspace_size(pc) == sa.sa_forward_workspace_size(pb) + 256
    lib = sa.load_library()
    f = sa.make_problem(4, 8, 64, 32, 10_000, dtype="bf16")
    fc = sa.make_problem(4, 8, 64, 32, 10_000, dtype="bf16", flags=sa.SA_FLAG_CHECK_OFFSETS)
    assert lib.sa_forward_fused_proj_workspace_size(ctypes.byref(fc), 256) == \
        lib.sa_forward_fused_proj_workspace_size(ctypes.byref(f), 256) + 256
    r = sa.make_problem(4, 8, 64, 32, 10_000, dtype="bf16", flags=sa.SA_FLAG_CHECK_OFFSETS)
    assert sa.sa_refine_workspace_size(r, 256, 2) == 0 and "flags" in sa.sa_last_error()
    assert sa.sa_backward_workspace_size(pc) == 0 and "flags" in sa.sa_last_error()
    g = sa.make_problem(4, 8, 128, 64, 10_000, dtype="bf16", flags=sa.SA_FLAG_BF16_GRADS)
    assert sa.sa_backward_workspace_size(g) > 0
    assert sa.sa_forward_workspace_size(g) == 0 and "flags" in sa.sa_last_error()


@pytest.mark.parametrize("cu,total,bits,first", [
    ([0, 10, 20, 30], 30, 0, -1),
    ([0], 0, 0, -1),
    ([5, 5, 5], 5, 0, -1),
    ([-1, 10, 20], 30, 1, 0),
    ([0, 10, 5, 30], 30, 2, 1),
    ([0, 10, 20, 31], 30, 4, 3),
    ([3, 2, 9], 8, 6, 0),
    ([-4, -5, 40], 30, 7, 0),
    ([0, 10, 20, 15, 30, 2], 100, 2, 2),
])
def test_check_offsets_rules_on_host(cu, total, bits, first):
    """The rules the device check applies (same rule code): bit 1 a negative
    first offset, bit 2 a decreasing pair, bit 4 an end past total_rows; the
    index is the first entry that breaks any rule."""
    assert sa.sa_check_offsets_host(cu, total) == (bits, first)
