"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds (several tiles,
ragged tails) and, for the large workloads, at full size on sampled outputs.

Bars: fp32 inputs max|g-o|/max|o| <= 1e-5; bf16 inputs relative L2 <= 1e-2
(oracle fed the same bf16 tensors).  Offsets and masks are checked
bit-exactly: NaN-poisoned rows outside users or masked change nothing,
packed == dense+lengths, an all-ones mask == no mask, two runs are equal."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_lse, assert_parity, rel_l2, run, to_dev, device
import sketch_attention_flashsa_amd as sa

pytestmark = pytest.mark.gpu


def _oracle(w, norm="history", mask=None, lengths_ok=True):
    msk = mask if mask is not None else w.get("mask")
    if w["layout"] == "packed":
        return oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=msk, norm=norm)
    return oracle.forward(w["P"], w["K"], w["V"], lengths=w["lengths"] if lengths_ok else None, mask=msk, norm=norm)


# ----------------------------------------------------------- named workloads
def test_tiny_fp32_workload_full():
    """B=1, L=1000, H=1, m=16, dh=32, fp32 -- the whole workload."""
    w = W.make(1)
    S, lse = run(w)
    So, lo = _oracle(w)
    assert_parity(S, So, "f32", "tiny fp32")
    assert_lse(lse, lo, "f32", "tiny fp32")


@pytest.mark.parametrize("cfg,B,max_len", [(2, 4, None), (3, 8, 6000), (4, 2, 3000)])
def test_bf16_workloads_reduced(cfg, B, max_len):
    """The bf16 workloads with fewer users / capped lengths, full oracle."""
    w = W.make(cfg, B=B, max_len=max_len)
    S, lse = run(w)
    So, lo = _oracle(w)
    assert_parity(S, So, "bf16", f"workload {cfg}")
    assert_lse(lse, lo, "bf16", f"workload {cfg}")


def _sample_bhj(w, n, rng):
    B, H, m = w["B"], w["H"], w["m"]
    L = w["lengths"].numpy()
    users = list(np.argsort(L)[:2]) + list(np.argsort(L)[-2:]) + list(rng.integers(0, B, size=n))
    out = []
    for b in users[:n]:
        out.append((int(b), int(rng.integers(0, H)), int(rng.integers(0, m))))
    return out


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_bf16_workloads_full_size_sampled(cfg):
    """Full-size workloads in the launch configuration the benchmark times;
    the oracle computes sampled (user, head, prototype) rows one by one."""
    w = W.make(cfg)
    S, lse = run(w)
    rng = np.random.default_rng(cfg)
    bhj = _sample_bhj(w, 24, rng)
    if w["layout"] == "packed":
        o, lo = oracle.forward_sample(w["P"], w["K"], w["V"], bhj, cu_offsets=w["cu_offsets"])
    else:
        o, lo = oracle.forward_sample(w["P"], w["K"], w["V"], bhj, lengths=w["lengths"])
    g = np.stack([S[b, h, j] for b, h, j in bhj])
    gl = np.array([lse[b, h, j] for b, h, j in bhj])
    assert_parity(g, o, "bf16", f"workload {cfg} sampled")
    assert_lse(gl, lo, "bf16", f"workload {cfg} sampled")
    assert np.all(np.isfinite(S))
    # users of length 1 (workload 3) reproduce their single value row exactly
    cu = w.get("cu_offsets")
    if cu is not None:
        for b in np.nonzero(w["lengths"].numpy() == 1)[0]:
            row = w["V"][int(cu[b])].double().numpy()              # [H, dh]
            assert np.array_equal(S[b], np.broadcast_to(row[:, None, :], S[b].shape)), "L=1 user must be exact"


# ------------------------------------------------------------- edge cases
RAGGED = [0, 1, 2, 31, 32, 33, 65, 700]


@pytest.mark.parametrize("dtype,H,m,dh", [("bf16", 4, 64, 32), ("bf16", 2, 128, 64), ("bf16", 3, 48, 32),
                                          ("bf16", 1, 32, 128), ("f32", 2, 16, 32), ("f32", 1, 300, 64),
                                          ("f32", 2, 8, 16)])
@pytest.mark.parametrize("norm", ["history", "prototype"])
def test_ragged_edges(dtype, H, m, dh, norm):
    """Empty users, L = 1, 2, tile-boundary lengths and a long tail."""
    w = W.random_case(101, B=len(RAGGED), H=H, m=m, dh=dh, lengths=RAGGED, dtype=dtype)
    S, lse = run(w, norm=norm)
    So, lo = _oracle(w, norm=norm)
    assert_parity(S, So, dtype, f"ragged {dtype} {norm}")
    assert_lse(lse, lo, dtype, f"ragged {dtype} {norm}")
    assert np.all(S[0] == 0), "empty user must give zeros"
    if norm == "history":
        assert np.all(np.isneginf(lse[0])), "empty user must give lse = -inf"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_chunks_many_segments(dtype):
    """A fixed small chunk size splits users over many segments; the merge
    must still agree with the oracle."""
    w = W.random_case(102, B=3, H=2, m=32, dh=32, lengths=[1000, 37, 2049], dtype=dtype)
    S, lse = run(w, chunk_rows=64)
    So, lo = _oracle(w)
    assert_parity(S, So, dtype, "chunk_rows=64")
    assert_lse(lse, lo, dtype, "chunk_rows=64")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mask_poisoned_rows_bit_exact(dtype):
    """Masked rows and rows outside every user, filled with NaN/Inf, change
    nothing bitwise; an all-ones mask equals no mask bitwise; masked results
    match the oracle."""
    w = W.random_case(103, B=4, H=2, m=32, dh=32, lengths=[300, 0, 77, 129], dtype=dtype, mask_p=0.3)
    S_ref, l_ref = run(w)
    So, lo = _oracle(w)
    assert_parity(S_ref, So, dtype, "masked")
    assert_lse(l_ref, lo, dtype, "masked")
    # poison masked rows
    w2 = dict(w)
    K, V = w["K"].clone(), w["V"].clone()
    bad = ~w["mask"].bool()
    K[bad] = float("nan")
    V[bad] = float("inf")
    w2["K"], w2["V"] = K, V
    S2, l2 = run(w2)
    assert np.array_equal(S2, S_ref) and np.array_equal(l2, l_ref), "masked rows must not leak"
    # rows outside every user: pad the buffer front and back with NaN
    pad = 40
    K3 = torch.full((pad + K.shape[0] + pad, 2, 32), float("nan"), dtype=K.dtype)
    V3 = K3.clone()
    K3[pad:pad + K.shape[0]] = w["K"]
    V3[pad:pad + V.shape[0]] = w["V"]
    mk3 = torch.zeros(K3.shape[0], dtype=torch.uint8)
    mk3[pad:pad + K.shape[0]] = w["mask"]
    w3 = dict(w, K=K3, V=V3, cu_offsets=w["cu_offsets"] + pad)
    S3, l3 = run(w3, mask=mk3)
    assert np.array_equal(S3, S_ref) and np.array_equal(l3, l_ref), "rows outside users must not leak"
    # all-ones mask == no mask
    w4 = dict(w)
    w4.pop("mask")
    S4, _ = run(w4)
    S5, _ = run(w4, mask=torch.ones(w["K"].shape[0], dtype=torch.uint8))
    assert np.array_equal(S4, S5), "all-ones mask must equal no mask"


@pytest.mark.parametrize("H,m,dh", [(8, 128, 64), (8, 64, 32), (1, 256, 128)])
@pytest.mark.parametrize("norm", ["history", "prototype"])
def test_streaming_kernel_masks_bit_exact(H, m, dh, norm):
    """The same properties on shapes the streaming kernel serves (its masked
    instances carry the mask bytes in the ring): masked rows match the oracle,
    NaN/Inf in masked rows change nothing bitwise, an all-ones mask equals no
    mask bitwise.  Ragged users put masked rows in segment tails too."""
    lengths = [700, 1, 33, 1000, 64, 0, 95]
    w = W.random_case(120 + dh, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16", mask_p=0.3)
    pb = sa.make_problem(w["B"], H, m, dh, w["K"].shape[0], dtype="bf16", norm=norm)
    expect = {("history", False): "sa_bf16_stream_kernel", ("history", True): "sa_bf16_stream_d128_kernel",
              ("prototype", False): "sa_proto_stream_kernel", ("prototype", True): "sa_bf16_stream_kernel"}
    assert sa.sa_forward_kernel_name(pb) == expect[(norm, dh == 128)]
    S_ref, l_ref = run(w, norm=norm)
    So, lo = _oracle(w, norm=norm)
    assert_parity(S_ref, So, "bf16", f"streaming masked {norm} dh={dh}")
    assert_lse(l_ref.reshape(lo.shape), lo, "bf16", f"streaming masked {norm} dh={dh}")
    bad = ~w["mask"].bool()
    K, V = w["K"].clone(), w["V"].clone()
    K[bad] = float("nan")
    V[bad] = float("inf")
    S2, l2 = run(dict(w, K=K, V=V), norm=norm)
    assert np.array_equal(S2, S_ref), "masked rows must not leak"
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(l2)) and np.array_equal(l2[fin], l_ref[fin])
    w4 = dict(w)
    w4.pop("mask")
    S4, _ = run(w4, norm=norm)
    S5, _ = run(w4, norm=norm, mask=torch.ones(w["K"].shape[0], dtype=torch.uint8))
    assert np.array_equal(S4, S5), "all-ones mask must equal no mask"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_equals_dense_bitwise(dtype):
    lengths = [500, 3, 0, 1200, 64]
    wp = W.random_case(104, B=5, H=4, m=64, dh=32, lengths=lengths, dtype=dtype, layout="packed")
    wd = W.random_case(104, B=5, H=4, m=64, dh=32, lengths=lengths, dtype=dtype, layout="dense")
    Sp, lp = run(wp)
    Sd, ld = run(wd)
    assert np.array_equal(Sp, Sd) and np.array_equal(lp, ld), "packed and dense+lengths must agree bitwise"
    # dense padding filled with NaN changes nothing
    K, V = wd["K"].clone(), wd["V"].clone()
    for b, n in enumerate(lengths):
        K[b, n:] = float("nan")
        V[b, n:] = float("nan")
    Sn, _ = run(dict(wd, K=K, V=V))
    assert np.array_equal(Sn, Sd), "dense padding must not leak"


def test_uneven_row_split():
    """About 118K rows (H=8, m=128, dh=64, bf16): enough rows that the
    streaming kernel gives the first half of its row ranges a larger share
    (R1 > R2), so ranges straddle user boundaries at uneven places.  Checked
    against the oracle, against the uniform split (same values to tolerance,
    different segments), and packed against dense+lengths bitwise."""
    lengths = [30011, 1, 0, 20000, 17, 19968, 12345, 511, 9000, 20000, 6992]
    wp = W.random_case(106, B=len(lengths), H=8, m=128, dh=64, lengths=lengths, dtype="bf16", layout="packed")
    S, lse = run(wp)
    So, lo = _oracle(wp)
    assert_parity(S, So, "bf16", "uneven row split")
    assert_lse(lse, lo, "bf16", "uneven row split")
    sa.sa_set_tuning(range_split=50)
    try:
        Su, lu = run(wp)
    finally:
        sa.sa_set_tuning()
    assert_parity(Su, So, "bf16", "uniform row split")
    assert not np.array_equal(S, Su), "the default split should segment these users differently"
    wd = W.random_case(106, B=len(lengths), H=8, m=128, dh=64, lengths=lengths, dtype="bf16", layout="dense")
    Sd, ld = run(wd)
    assert np.array_equal(S, Sd) and np.array_equal(lse, ld), "packed and dense+lengths must agree bitwise"


@pytest.mark.parametrize("H,m", [(1, 1024), (2, 256), (3, 512)])
def test_dh128_streaming(H, m):
    """dh = 128 with m a multiple of 256 runs the streaming kernel with m / 256
    blocks per head: ragged users, a mask, packed == dense bitwise."""
    lengths = [900, 0, 1, 31, 33, 257, 1500]
    w = W.random_case(107 + m + H, B=len(lengths), H=H, m=m, dh=128, lengths=lengths, dtype="bf16", mask_p=0.2)
    assert sa.sa_forward_kernel_name(sa.make_problem(len(lengths), H, m, 128, int(sum(lengths)))) == \
        "sa_bf16_stream_d128_kernel"
    S, lse = run(w)
    So, lo = _oracle(w)
    assert_parity(S, So, "bf16", f"dh=128 H={H} m={m}")
    assert_lse(lse, lo, "bf16", f"dh=128 H={H} m={m}")
    wd = W.random_case(107 + m + H, B=len(lengths), H=H, m=m, dh=128, lengths=lengths, dtype="bf16", layout="dense")
    wp = W.random_case(107 + m + H, B=len(lengths), H=H, m=m, dh=128, lengths=lengths, dtype="bf16")
    Sp, lp = run(wp)
    Sd, ld = run(wd)
    assert np.array_equal(Sp, Sd) and np.array_equal(lp, ld), "packed and dense+lengths must agree bitwise"


def test_deterministic_and_isolated():
    w = W.random_case(105, B=3, H=2, m=64, dh=64, lengths=[3000, 1500, 2500], dtype="bf16")
    S1, l1 = run(w)
    S2, l2 = run(w)
    assert np.array_equal(S1, S2) and np.array_equal(l1, l2), "two runs must be bitwise equal"
    K = w["K"].clone()
    cu = w["cu_offsets"].tolist()
    K[cu[2]:cu[3]] = -K[cu[2]:cu[3]]
    S3, _ = run(dict(w, K=K))
    assert np.array_equal(S3[:2], S1[:2]) and not np.array_equal(S3[2], S1[2]), "users must not interact"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_p_zero_gives_mean(dtype):
    w = W.random_case(106, B=2, H=2, m=16, dh=32, lengths=[999, 45], dtype=dtype)
    w["P"] = torch.zeros_like(w["P"])
    S, _ = run(w)
    cu = w["cu_offsets"].tolist()
    for b in range(2):
        mean = w["V"][cu[b]:cu[b + 1]].double().mean(dim=0).numpy()     # [H, dh]
        assert_parity(S[b], np.broadcast_to(mean[:, None, :], S[b].shape), dtype, "P=0 mean")


@pytest.mark.parametrize("scale_p,offset", [(4.0, 0.0), (1.0, 80.0), (1.0, -200.0), (8.0, 120.0)])
def test_peaked_and_shifted_scores(scale_p, offset):
    """Peaked rows (P scaled up) and large constant score offsets neither
    overflow nor lose accuracy.  The offset is exact: channel 0 of every
    prototype is set to 4 and channel 0 of every key row is shifted by
    offset*sqrt(dh)/4, so every score moves by about `offset` (past the fp32
    exp range for |offset| >= 89)."""
    dh = 32
    w = W.random_case(107, B=2, H=2, m=32, dh=dh, lengths=[4000, 777], dtype="bf16")
    P = w["P"].float() * scale_p
    K = w["K"].float()
    if offset:
        P[:, :, 0] = 4.0
        K[:, :, 0] += offset * np.sqrt(dh) / 4.0
    w = dict(w, P=P.to(torch.bfloat16), K=K.to(torch.bfloat16))
    S, lse = run(w)
    So, lo = _oracle(w)
    assert np.all(np.isfinite(S))
    assert_parity(S, So, "bf16", f"peaked x{scale_p} offset {offset}")
    assert_lse(lse, lo, "bf16", f"peaked x{scale_p} offset {offset}")


@pytest.mark.parametrize("ramp,masked,unit_scale", [(0.0, False, True), (1.0, False, True), (-1.0, False, True),
                                                    (1.0, True, True), (1.0, False, False), (1.0, True, False)])
def test_dh128_pipeline_segments_and_moving_maximum(ramp, masked, unit_scale):
    """The dh = 128 kernel forms a stage's weights while the next stage's
    score products run, shifting those products when the weights move the
    running maximum.  Segments of 1 .. 14 stages (every remainder of the
    six-slot ring, ragged tails) and a score ramp along the rows: channel 0 of
    every prototype is 4 and channel 0 of key row r is ramp * r / 4, so base-2
    scores move by about `ramp` per row (the maximum moves in almost every
    stage when ramp > 0, never after the first when ramp < 0).  unit_scale:
    the float nearest 1 / log2(e), for which scale * log2(e) is exactly 1 in
    float, so the pre-scaled prototypes are exact; else the default
    1 / sqrt(dh), where the requested lse makes the kernel scale unrounded
    products.  Either way scores of several hundred meet the lse bar."""
    dh, m = 128, 256
    unit = float(np.float32(1.0) / np.float32(np.log2(np.e))) if unit_scale else 1.0 / np.sqrt(dh)
    lengths = [1, 32, 33, 64, 95, 160, 191, 192, 193, 224, 385, 448]
    w = W.random_case(131 + int(ramp * 10) + masked, B=len(lengths), H=1, m=m, dh=dh, lengths=lengths,
                      dtype="bf16", mask_p=0.2 if masked else 0.0)
    P = w["P"].float()
    K = w["K"].float()
    if ramp:
        P[:, :, 0] = 4.0
        cu = w["cu_offsets"].tolist()
        for b in range(len(lengths)):
            r = torch.arange(cu[b + 1] - cu[b], dtype=torch.float32)
            K[cu[b]:cu[b + 1], :, 0] = (ramp * r / 4.0 / (unit * np.log2(np.e)))[:, None]
    w = dict(w, P=P.to(torch.bfloat16), K=K.to(torch.bfloat16))
    assert sa.sa_forward_kernel_name(sa.make_problem(len(lengths), 1, m, dh, int(sum(lengths)))) == \
        "sa_bf16_stream_d128_kernel"
    So, lo = oracle.forward(w["P"], w["K"], w["V"], cu_offsets=w["cu_offsets"], mask=w.get("mask"), scale=unit)
    for chunk in (0, 96):
        S, lse = run(w, chunk_rows=chunk, scale=unit)
        assert np.all(np.isfinite(S))
        assert_parity(S, So, "bf16", f"dh=128 ramp {ramp} masked {masked} chunk {chunk}")
        assert_lse(lse, lo, "bf16", f"dh=128 ramp {ramp} masked {masked} chunk {chunk}")


@pytest.mark.parametrize("H,m,dh,mask_p", [(8, 128, 64, 0.0), (8, 64, 32, 0.0), (1, 256, 128, 0.0),
                                            (8, 128, 64, 0.3), (1, 256, 128, 0.3)])
def test_streaming_lse_with_large_scores(H, m, dh, mask_p):
    """Scores of several hundred on the streaming kernels' shapes at the
    default scale: with the lse requested the kernels scale unrounded
    products (a prototype rounded once to bf16 after scaling would shift its
    lse by about 2^-9 of the scores), so lse meets its bar; S computed with
    and without the lse agrees to the bf16 bar."""
    lengths = [700, 33, 1300, 1]
    w = W.random_case(141 + dh + m, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16", mask_p=mask_p)
    P = w["P"].float()
    K = w["K"].float()
    P[:, :, 0] = 4.0
    cu = w["cu_offsets"].tolist()
    for b in range(len(lengths)):
        r = torch.arange(cu[b + 1] - cu[b], dtype=torch.float32)
        K[cu[b]:cu[b + 1], :, 0] = (0.5 * r * np.sqrt(dh) / 4.0)[:, None]   # scores up to ~650
    w = dict(w, P=P.to(torch.bfloat16), K=K.to(torch.bfloat16))
    assert sa.sa_forward_kernel_name(sa.make_problem(len(lengths), H, m, dh, int(sum(lengths)))).startswith(
        "sa_bf16_stream")
    S, lse = run(w)
    So, lo = _oracle(w)
    assert_parity(S, So, "bf16", f"large scores H={H} m={m} dh={dh}")
    assert_lse(lse, lo, "bf16", f"large scores H={H} m={m} dh={dh}")
    d = to_dev(w, device())
    S2 = sa.sa_forward(d["P"], d["K"], d["V"], cu_offsets=d["cu_offsets"],
                       mask=d.get("mask"))
    torch.cuda.synchronize()
    assert_parity(S2.double().cpu().numpy(), So, "bf16", f"large scores without lse H={H} m={m} dh={dh}")


@pytest.mark.parametrize("H,m,dh", [(2, 32, 32), (8, 128, 64), (3, 48, 32), (1, 256, 128)])
def test_per_user_prototypes(H, m, dh):
    """P [B, H, m, dh] (stacked refinement feeds per-user queries) against the
    oracle with the same per-user sets, on the streaming kernel's shapes and a
    register-staged one; and each user equals a shared-P call with that
    user's prototypes, bitwise."""
    w = W.random_case(108 + m, B=4, H=H, m=m, dh=dh, lengths=[700, 1, 0, 1300], dtype="bf16")
    Pu = torch.stack([w["P"], -w["P"], w["P"].flip(-1), 0.5 * w["P"]]).to(torch.bfloat16)
    S, lse = run(dict(w, P=Pu))
    So, lo = oracle.forward(Pu, w["K"], w["V"], cu_offsets=w["cu_offsets"])
    assert_parity(S, So, "bf16", f"per-user prototypes H={H} m={m} dh={dh}")
    assert_lse(lse, lo, "bf16", f"per-user prototypes H={H} m={m} dh={dh}")
    for b in (0, 1, 3):
        Sb, _ = run(dict(w, P=Pu[b]))
        assert np.array_equal(S[b], Sb[b]), "per-user prototypes must match the shared call"


# --------------------------------------------------------- prototype axis
@pytest.mark.parametrize("cfg,B,max_len", [(1, None, None), (2, 2, 4000), (3, 6, 3000), (4, 2, 2000)])
def test_prototype_axis_workloads(cfg, B, max_len):
    w = W.make(cfg, B=B, max_len=max_len)
    S, lse = run(w, norm="prototype")
    So, lo = _oracle(w, norm="prototype")
    dt = w["dtype"]
    assert_parity(S, So, dt, f"prototype axis, workload {cfg}")
    rows = lo.shape[0]
    assert_lse(lse.reshape(rows, -1), lo, dt, f"prototype axis lse, workload {cfg}")


def test_prototype_axis_full_size_sampled():
    """The 100K workload on the prototype axis in the launch configuration
    the benchmark times: one whole user (100,000 rows) against the oracle run
    on that user alone, and the per-row normalisers of sampled rows of every
    user against the oracle run on each row alone."""
    w = W.make(4)
    S, lse = run(w, norm="prototype")
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(lse))
    cu = w["cu_offsets"].numpy()
    H = w["H"]
    lse = lse.reshape(-1, H)
    b = w["B"] - 1
    lo_, hi_ = int(cu[b]), int(cu[b + 1])
    one = torch.tensor([0, hi_ - lo_], dtype=torch.int32)
    So, lo = oracle.forward(w["P"], w["K"][lo_:hi_], w["V"][lo_:hi_], cu_offsets=one, norm="prototype")
    assert_parity(S[b], So[0], "bf16", f"prototype axis, user {b} of the 100K workload")
    assert_lse(lse[lo_:hi_], lo, "bf16", f"prototype axis lse, user {b}")
    rng = np.random.default_rng(44)
    rows = [int(cu[u]) + int(rng.integers(0, cu[u + 1] - cu[u])) for u in range(w["B"]) for _ in range(2)]
    single = torch.tensor([0, 1], dtype=torch.int32)
    for r in rows:
        _, lr = oracle.forward(w["P"], w["K"][r:r + 1], w["V"][r:r + 1], cu_offsets=single, norm="prototype")
        assert_lse(lse[r:r + 1], lr, "bf16", f"prototype axis lse, row {r}")


def _s_only(w, norm="prototype"):
    """S from a call that passes no lse output (the kernel instances that
    write no row normalisers)."""
    d = to_dev(w, device())
    S = sa.sa_forward(d["P"], d["K"], d["V"], cu_offsets=d["cu_offsets"], mask=d.get("mask"), norm=norm)
    torch.cuda.synchronize()
    return S.double().cpu().numpy()


@pytest.mark.parametrize("H,m,dh,waves", [(8, 128, 64, 8), (2, 128, 64, 8), (4, 64, 64, 8), (4, 64, 32, 8),
                                          (8, 32, 32, 8), (8, 128, 64, 16), (8, 64, 32, 16)])
@pytest.mark.parametrize("masked", [False, True])
def test_prototype_one_pass_shapes(H, m, dh, waves, masked):
    """Every block shape of the one-pass prototype-axis kernel (8- and
    16-wave blocks; 1, 2 and 4 prototype blocks per head), ragged users,
    with and without a mask: S against the oracle from a call without lse
    (pre-scaled prototypes) and from one with lse (exact prototypes), lse
    against the oracle."""
    lengths = [700, 1, 33, 0, 1000, 64, 95, 31]
    w = W.random_case(130 + m + dh + H, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16",
                      mask_p=0.25 if masked else 0.0)
    sa.sa_set_tuning(stream_waves=waves)
    try:
        pb = sa.make_problem(w["B"], H, m, dh, w["K"].shape[0], dtype="bf16", norm="prototype")
        assert sa.sa_forward_kernel_name(pb) == "sa_proto_stream_kernel"
        S1 = _s_only(w)
        S, lse = run(w, norm="prototype")
    finally:
        sa.sa_set_tuning()
    So, lo = _oracle(w, norm="prototype")
    tag = f"one pass H={H} m={m} dh={dh} waves={waves} masked={masked}"
    assert_parity(S1, So, "bf16", tag + " (no lse)")
    assert_parity(S, So, "bf16", tag)
    assert_lse(lse.reshape(lo.shape), lo, "bf16", tag)
    # the instance without lse pre-scales P (one more bf16 rounding): the two
    # agree to the bf16 bar, not bitwise
    assert rel_l2(S1, S) < 1e-2, f"{tag}: S with and without lse differ by {rel_l2(S1, S):.2e}"


@pytest.mark.parametrize("offset", [50.0, 120.0, -200.0])
def test_prototype_exact_path(offset):
    """Rows whose scores all move by `offset` (channel 0 of every prototype
    set to 4, channel 0 of the key shifted by offset*sqrt(dh)/4): their
    partial row sums leave [2^-60, 2^60] (2^72 at +50, past the fp32 range at
    +120 and -200), so the stages that hold them take the exact path.  The
    shifted rows come in blocks of 96, so fast and exact stages alternate
    inside one segment; within a row the offset cancels, the normaliser
    carries it."""
    H, m, dh = 8, 128, 64
    lengths = [3000, 1, 0, 700, 40]
    w = W.random_case(140, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16")
    P = w["P"].float()
    K = w["K"].float()
    P[:, :, 0] = 4.0
    shifted = (torch.arange(K.shape[0]) // 96) % 2 == 1
    K[shifted, :, 0] += offset * np.sqrt(dh) / 4.0
    w = dict(w, P=P.to(torch.bfloat16), K=K.to(torch.bfloat16))
    S1 = _s_only(w)
    S, lse = run(w, norm="prototype")
    So, lo = _oracle(w, norm="prototype")
    assert np.all(np.isfinite(S))
    assert_parity(S1, So, "bf16", f"exact path offset {offset} (no lse)")
    assert_parity(S, So, "bf16", f"exact path offset {offset}")
    assert_lse(lse.reshape(lo.shape), lo, "bf16", f"exact path offset {offset}")
    assert rel_l2(S1, S) < 1e-2


def test_prototype_axis_masked_and_dense():
    w = W.random_case(109, B=3, H=2, m=64, dh=64, lengths=[600, 0, 130], dtype="bf16", layout="dense", mask_p=0.2)
    S, lse = run(w, norm="prototype")
    So, lo = _oracle(w, norm="prototype")
    assert_parity(S, So, "bf16", "prototype masked dense")
    assert_lse(lse, lo, "bf16", "prototype masked dense")


@pytest.mark.parametrize("H,m,dh", [(8, 128, 64), (4, 64, 32), (1, 1024, 128)])
@pytest.mark.parametrize("masked", [False, True])
def test_same_buffer_keys_and_values(H, m, dh, masked):
    """K and V given as one buffer (as the production shape's folded path
    passes X for both): the oracle with V = K, and bitwise the same result as
    two separate copies."""
    lengths = [900, 0, 1, 31, 33, 257, 1500]
    w = W.random_case(150 + m + dh, B=len(lengths), H=H, m=m, dh=dh, lengths=lengths, dtype="bf16",
                      mask_p=0.2 if masked else 0.0)
    w = dict(w, V=w["K"])
    d = to_dev(w, device())
    S1, l1 = sa.sa_forward(d["P"], d["K"], d["K"], cu_offsets=d["cu_offsets"], mask=d.get("mask"), return_lse=True)
    S2, l2 = sa.sa_forward(d["P"], d["K"], d["K"].clone(), cu_offsets=d["cu_offsets"], mask=d.get("mask"),
                           return_lse=True)
    torch.cuda.synchronize()
    S1, l1, S2, l2 = (x.double().cpu().numpy() for x in (S1, l1, S2, l2))
    So, lo = _oracle(w)
    assert_parity(S1, So, "bf16", f"K = V buffer H={H} m={m} dh={dh}")
    assert_lse(l1, lo, "bf16", f"K = V buffer H={H} m={m} dh={dh}")
    assert np.array_equal(S1, S2) and np.array_equal(l1, l2), "one copy of K = V must equal two copies"
