// sa_api.hip -- host side of the libsketchattn C ABI (include/sketchattn.h):
// argument validation, work split, workspace layout and kernel dispatch.
// Nothing here reads device memory or synchronises; every launch goes to the
// caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sa_internal.h"
#include "sa_fold.h"
#include "sa_proto.h"
#include "sa_stream_d128.h"
#include "sketchattn.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
thread_local sa_tuning g_tune = {};

// The timing events of a call: taken (and forgotten) at the top of every
// compute entry point, before anything can fail.
struct Events {
    hipEvent_t start, stop;
};
Events take_events() {
    const Events ev{g_ev_start, g_ev_stop};
    g_ev_start = g_ev_stop = nullptr;
    return ev;
}

// A launch reports its error through the runtime's per-thread "last error",
// which an earlier, unrelated HIP call may have left set: clear it first, so
// that a call's status reflects its own launches only.  (Errors that poison
// the device context persist in the runtime and still fail the launches.)
void clear_stale_error() { (void)hipGetLastError(); }

sa_status fail(sa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

struct DeviceInfo {
    int cus = 256;
    size_t lds = 65536;
};

DeviceInfo device_info() {
    static std::mutex mu;
    static DeviceInfo cache[64];
    static bool known[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{};
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev]) {
        int cus = 0, lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cache[dev].cus = cus;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && lds > 0)
            cache[dev].lds = (size_t)lds;
        known[dev] = true;
    }
    return cache[dev];
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int kRowMinBf16 = 512;   // smallest automatic segment (rows)
constexpr int kRowMinF32 = 128;
// Share (percent) of the rows that the first half of the streaming kernel's
// row ranges takes when two of its blocks share a CU (measured on MI355X).
constexpr int kStreamSplit = 64;
// Grid of the backward's dK/dV kernel, in blocks per CU (row ranges x heads;
// two of its 4-wave blocks are resident per CU at dh = 64, so larger grids
// run in rounds).  With fp32 gradients at dh = 64 one block per CU: on the
// 100K workload the whole backward took 2.97-3.00 ms against 3.19-3.21 ms
// with four, the dK/dV kernel 2.13 against 2.25 ms (its 16-byte stores then
// come from fewer concurrent row streams); with bf16 gradients the sweeps
// disagreed with the profiled run, so four stays.
constexpr int kDkdvBlocksPerCu = 4;
constexpr int kDkdvBlocksPerCuF32d64 = 1;

// Everything the dispatcher derives from the problem.
struct Plan {
    bool f32 = false;
    bool packed = true;
    int64_t buf_rows = 0;     // rows of the K/V buffers the kernels may address
    int G = 1;                // row-range blocks
    int R_fixed = 0, R_min = kRowMinBf16;
    int split = 50;           // RowSplit share of the first half of the ranges
    // fused entry, shapes outside the on-chip kernel: K = X Wk is projected
    // into the workspace (after the forward's own sections), then sa_forward
    bool two_pass = false;
    bool fold_keys = false;   // one head, dh == d_model: W_K folded into the prototypes, no K pass
    size_t off_kproj = 0, off_wt = 0, off_pfold = 0, fwd_total = 0;
    sa::Bf16Config cfg{};
    bool stream = false;      // bf16: the direct-to-LDS streaming kernel serves this shape
    bool proto1 = false;      // prototype axis in one pass (sa_proto_stream_kernel), no row-normaliser pass
    bool d128 = false;        // history axis, dh = 128: the pipelined streaming kernel (sa_stream_d128.hip)
    sa::StreamConfig scfg{};
    int groups = 1;           // bf16: unit groups per row range
    bool check_offsets = false;  // SA_FLAG_CHECK_OFFSETS: status section first
    // workspace layout (byte offsets)
    size_t off_status = 0, off_vcu = 0, off_M = 0, off_Z = 0, off_acc = 0, off_tok = 0, total = 0;
};

void set_layout(const sa_problem* pb, Plan* pl);

// Validation and work split shared by every entry point.  The workspace size
// depends only on the problem description, never on which optional pointers
// a call passes, so the size query and the call always agree.  `flags_ok`
// are the sa_problem.flags bits the calling entry point accepts.
sa_status make_plan(const sa_problem* pb, bool packed, Plan* pl, int32_t flags_ok = SA_FLAG_CHECK_OFFSETS) {
    if (!pb) return fail(SA_ERR_INVALID_ARG, "problem is NULL");
    if (pb->B < 0 || pb->H < 1 || pb->m < 1 || pb->dh < 1)
        return fail(SA_ERR_INVALID_ARG, "need B >= 0, H >= 1, m >= 1, dh >= 1 (got B=%d H=%d m=%d dh=%d)", pb->B,
                    pb->H, pb->m, pb->dh);
    if (pb->dtype != SA_DTYPE_F32 && pb->dtype != SA_DTYPE_BF16)
        return fail(SA_ERR_INVALID_ARG, "unknown dtype %d", pb->dtype);
    if (pb->norm != SA_NORM_HISTORY && pb->norm != SA_NORM_PROTOTYPE)
        return fail(SA_ERR_INVALID_ARG, "unknown norm %d", pb->norm);
    if (pb->flags & ~flags_ok)
        return fail(SA_ERR_INVALID_ARG, "flags %d: this entry point accepts only the bits %d", pb->flags, flags_ok);
    pl->check_offsets = (pb->flags & SA_FLAG_CHECK_OFFSETS) != 0;
    if (pb->total_rows < 0 || pb->total_rows > INT32_MAX)
        return fail(SA_ERR_INVALID_ARG, "total_rows must be in [0, 2^31)");
    if (pb->chunk_rows < 0 || pb->chunk_rows % sa::kRowAlign != 0)
        return fail(SA_ERR_INVALID_ARG, "chunk_rows must be 0 or a positive multiple of %d", sa::kRowAlign);
    if (!(pb->scale >= 0.f) || isinf(pb->scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite and >= 0");
    const int64_t hd = (int64_t)pb->H * pb->dh;
    if ((pb->k_row_stride != 0 && pb->k_row_stride < hd) || (pb->v_row_stride != 0 && pb->v_row_stride < hd))
        return fail(SA_ERR_INVALID_ARG, "row strides must be 0 or >= H*dh");
    if (pb->q_batch_stride < 0) return fail(SA_ERR_INVALID_ARG, "q_batch_stride must be >= 0");
    if (pb->q_batch_stride != 0 && pb->q_batch_stride < (int64_t)pb->H * pb->m * pb->dh)
        return fail(SA_ERR_INVALID_ARG, "q_batch_stride must be 0 or >= H*m*dh");
    if ((int64_t)pb->H * pb->m * pb->dh > INT32_MAX) return fail(SA_ERR_INVALID_ARG, "H*m*dh too large");

    pl->f32 = pb->dtype == SA_DTYPE_F32;
    pl->packed = packed;
    if (pb->L_max < 0) return fail(SA_ERR_INVALID_ARG, "L_max must be >= 0");
    if (packed && pb->L_max != 0) return fail(SA_ERR_INVALID_ARG, "L_max must be 0 with cu_offsets");
    const int64_t need = (int64_t)pb->B * pb->L_max;
    if (need > INT32_MAX) return fail(SA_ERR_INVALID_ARG, "B*L_max must be < 2^31");
    if (pb->L_max > 0 && pb->total_rows != 0 && pb->total_rows < need)
        return fail(SA_ERR_INVALID_ARG, "dense layout: total_rows (%lld) < B*L_max (%lld)",
                    (long long)pb->total_rows, (long long)need);
    pl->buf_rows = pb->total_rows > need ? pb->total_rows : need;
    if (pl->f32) {
        if (!(pb->dh == 16 || pb->dh == 32 || pb->dh == 64 || pb->dh == 128))
            return fail(SA_ERR_UNSUPPORTED, "f32: dh must be 16, 32, 64 or 128 (got %d)", pb->dh);
    } else {
        if (!(pb->dh == 32 || pb->dh == 64 || pb->dh == 128) || pb->m % 16 != 0)
            return fail(SA_ERR_UNSUPPORTED, "bf16: dh must be 32, 64 or 128 and m a multiple of 16 (got dh=%d m=%d)",
                        pb->dh, pb->m);
        if (!sa::bf16_config(pb->dh, pb->m, pb->H, device_info().lds, g_tune.bf16_tile_mb, g_tune.bf16_tile_nw,
                             &pl->cfg))
            return fail(SA_ERR_UNSUPPORTED, "bf16: tile needs %zu bytes of LDS, device allows %zu",
                        pl->cfg.lds_bytes, device_info().lds);
        const int64_t ks = pb->k_row_stride ? pb->k_row_stride : hd;
        const int64_t vs = pb->v_row_stride ? pb->v_row_stride : hd;
        if (ks % 8 != 0 || vs % 8 != 0 || pb->q_batch_stride % 8 != 0)
            return fail(SA_ERR_UNSUPPORTED, "bf16: row strides and q_batch_stride must be multiples of 8 elements");
    }

    const DeviceInfo dev = device_info();
    int per_row_range, blocks_per_cu;
    if (pl->f32) {
        per_row_range = pb->H * ((pb->m + 255) / 256);
        blocks_per_cu = 4;
        pl->R_min = kRowMinF32;
    } else {
        pl->stream =
            !g_tune.register_staged && sa::stream_config(pb->dh, pb->m, pb->H, g_tune.stream_waves, &pl->scfg);
        pl->proto1 = pl->stream && pb->norm == SA_NORM_PROTOTYPE && sa::proto_one_pass(pl->scfg, pb->dh);
        pl->d128 = pl->stream && pb->norm == SA_NORM_HISTORY && pb->dh == 128 &&
                   sa::stream_d128_config(pb->m, pb->H, &pl->scfg);
        if (pl->stream) {
            pl->groups = pl->scfg.groups;
            blocks_per_cu = pl->scfg.blocks_per_cu;
            // dh = 32 on the history axis: one block per CU (half the row
            // ranges, so half the segments, partial statistics and merge
            // inputs) took 6-7 % less kernel time and 10 % less per call than
            // two on the 10K-row and variable-length workloads; at dh = 64 two
            // stay faster down to 400K rows
            if (pb->dh == 32 && pb->norm == SA_NORM_HISTORY) blocks_per_cu = 1;
        } else {
            const int units = pb->H * (pb->m / pl->cfg.protos_per_wave);
            pl->groups = (units + pl->cfg.waves - 1) / pl->cfg.waves;
            blocks_per_cu = pl->cfg.blocks_per_cu;
        }
        per_row_range = pl->groups;
        pl->R_min = kRowMinBf16;
    }
    const int64_t rows_upper = pb->L_max > 0 ? need : pb->total_rows;
    if (pb->chunk_rows > 0) {
        pl->R_fixed = pb->chunk_rows;
        const int64_t G = (rows_upper + pb->chunk_rows - 1) / pb->chunk_rows;
        pl->G = (int)(G > 0 ? G : 1);
    } else {
        if (g_tune.blocks_per_cu > 0) blocks_per_cu = g_tune.blocks_per_cu;
        const int64_t G = (int64_t)dev.cus * blocks_per_cu / per_row_range;
        pl->G = (int)(G > 0 ? G : 1);
        // two streaming blocks per CU: the older one (first half of the
        // ranges in dispatch order) gets the larger share of the rows
        if (pl->stream && blocks_per_cu == 2) {
            pl->split = g_tune.range_split > 0 ? g_tune.range_split : kStreamSplit;
        }
    }

    set_layout(pb, pl);
    return SA_OK;
}

// Workspace layout for the plan's G (byte offsets, 256-byte aligned sections).
void set_layout(const sa_problem* pb, Plan* pl) {
    const size_t nslot = (size_t)pl->G + (size_t)pb->B;
    const size_t hm = (size_t)pb->H * pb->m;
    size_t off = 0;
    pl->off_status = off;
    if (pl->check_offsets) off = align_up(off + 2 * sizeof(int32_t));
    pl->off_vcu = off;
    off = align_up(off + sizeof(int32_t) * ((size_t)pb->B + 1));
    pl->off_M = off;
    off = align_up(off + sizeof(float) * nslot * hm);
    pl->off_Z = off;
    off = align_up(off + sizeof(float) * nslot * hm);
    pl->off_acc = off;
    off = align_up(off + sizeof(float) * nslot * hm * pb->dh);
    pl->off_tok = off;
    // the two-pass prototype axis keeps every row's normaliser between its passes
    if (pb->norm == SA_NORM_PROTOTYPE && !pl->proto1)
        off = align_up(off + sizeof(float) * (size_t)pl->buf_rows * pb->H);
    pl->total = off;
}

// Plan of the fused projection entry: the general validation (packed layout),
// the fused kernel's shape limits, and its own work split.
sa_status make_fused_plan(const sa_problem* pb, int32_t d_model, Plan* pl) {
    sa_status st = make_plan(pb, true, pl);
    if (st != SA_OK) return st;
    if (pb->dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "fused projection: bf16 inputs only");
    if (pb->norm != SA_NORM_HISTORY) return fail(SA_ERR_UNSUPPORTED, "fused projection: history axis only");
    if (d_model < 1) return fail(SA_ERR_INVALID_ARG, "d_model must be >= 1 (got %d)", d_model);
    if (!sa::fused_supported(d_model, pb->m, pb->dh)) {
        // two passes: the projection kernel, then the streaming forward on
        // K (workspace) and V = X; make_plan above planned that forward
        const int64_t hd = (int64_t)pb->H * pb->dh;
        if (pl->stream && pb->H == 1 && hd == d_model && pb->q_batch_stride == 0) {
            // one head as wide as the model: the scores are (P W_K^T) X^T,
            // so K is never formed; the workspace holds the folded prototypes
            pl->two_pass = true;
            pl->fold_keys = true;
            pl->fwd_total = pl->total;
            pl->off_pfold = align_up(pl->total);
            pl->total = align_up(pl->off_pfold + 2 * (size_t)pb->m * d_model);
            return SA_OK;
        }
        if (!(pl->stream && hd == d_model && sa::project_supported(d_model, (int)hd) && pb->q_batch_stride == 0))
            return fail(SA_ERR_UNSUPPORTED,
                        "fused projection: needs dh == 32, d_model in {128, 256}, m in {64, 128, 256}, or (two "
                        "passes) V = X with H*dh == d_model in {128, 256}, a streaming-kernel shape and shared P "
                        "(got dh=%d d_model=%d m=%d H=%d)", pb->dh, d_model, pb->m, pb->H);
        pl->two_pass = true;
        pl->fwd_total = pl->total;
        pl->off_kproj = align_up(pl->total);
        pl->off_wt = align_up(pl->off_kproj + 2 * (size_t)pl->buf_rows * hd);
        pl->total = align_up(pl->off_wt + 2 * (size_t)hd * d_model);
        return SA_OK;
    }
    if (pb->chunk_rows > 0) {
        pl->R_fixed = pb->chunk_rows;
        const int64_t G = (pb->total_rows + pb->chunk_rows - 1) / pb->chunk_rows;
        pl->G = (int)(G > 0 ? G : 1);
    } else {
        pl->R_fixed = 0;
        const int64_t G = (int64_t)device_info().cus / sa::fused_groups(pb->H);
        pl->G = (int)(G > 0 ? G : 1);
    }
    pl->R_min = kRowMinBf16;
    pl->split = 50;
    set_layout(pb, pl);
    return SA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

sa_status hip_fail(hipError_t e, const char* what) {
    return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t sa_forward_workspace_size(const sa_problem* pb) {
    Plan pl;
    if (!pb || make_plan(pb, pb->L_max == 0, &pl) != SA_OK) return 0;
    return pl.total;
}

const char* sa_forward_kernel_name(const sa_problem* pb) {
    Plan pl;
    if (!pb || make_plan(pb, pb->L_max == 0, &pl) != SA_OK) return nullptr;
    if (pl.f32) return "sa_f32_fwd_kernel";
    if (pl.proto1) return "sa_proto_stream_kernel";
    if (pl.d128) return "sa_bf16_stream_d128_kernel";
    return pl.stream ? "sa_bf16_stream_kernel" : "sa_bf16_fwd_kernel";
}

sa_status sa_forward(const sa_problem* pb, const void* P, const void* K, const void* V, const int32_t* cu_offsets,
                     const int32_t* lengths, const uint8_t* mask, float* S_out, float* lse_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    const Events ev = take_events();
    clear_stale_error();
    Plan pl;
    const bool packed = cu_offsets != nullptr;
    sa_status st = make_plan(pb, packed, &pl);
    if (st != SA_OK) return st;
    if (lengths && packed) return fail(SA_ERR_INVALID_ARG, "lengths is only valid for the dense layout");
    if (pb->B == 0) return SA_OK;
    if (!P || !K || !V || !S_out) return fail(SA_ERR_INVALID_ARG, "P, K, V and S_out must be non-NULL");
    const size_t el = pl.f32 ? 4 : 2;
    if (!pl.f32 && (!aligned(P, 16) || !aligned(K, 16) || !aligned(V, 16)))
        return fail(SA_ERR_INVALID_ARG, "bf16: P, K and V must be 16-byte aligned");
    if (!aligned(P, el) || !aligned(K, el) || !aligned(V, el) || !aligned(S_out, 16) || !aligned(lse_out, 4))
        return fail(SA_ERR_INVALID_ARG, "misaligned pointer");
    if (pl.total > 0 && (!workspace || workspace_bytes < pl.total))
        return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", pl.total, workspace_bytes);
    if (workspace && !aligned(workspace, kAlign)) return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    unsigned char* ws = (unsigned char*)workspace;
    sa::Users users{};
    users.cu = cu_offsets;
    users.vcu = nullptr;
    users.B = pb->B;
    users.L_max = pb->L_max;
    const int64_t hd = (int64_t)pb->H * pb->dh;
    const float scale = pb->scale > 0.f ? pb->scale : 1.0f / sqrtf((float)pb->dh);

    hipError_t e;
    const int32_t* status = nullptr;
    if (pl.check_offsets) {
        int32_t* sw = (int32_t*)(ws + pl.off_status);
        if ((e = sa::launch_check_offsets(cu_offsets, pb->B, pb->total_rows, sw, stream)) != hipSuccess)
            return hip_fail(e, "offsets check");
        status = sw;
    }
    if (!packed && lengths) {
        users.vcu = (int32_t*)(ws + pl.off_vcu);
        e = sa::launch_dense_vcu(lengths, pb->B, pb->L_max, (int32_t*)(ws + pl.off_vcu), stream);
        if (e != hipSuccess) return hip_fail(e, "dense offsets");
    }
    sa::Partials part{(float*)(ws + pl.off_acc), (float*)(ws + pl.off_M), (float*)(ws + pl.off_Z)};
    float* lse2_tok = (float*)(ws + pl.off_tok);

    if (pb->norm == SA_NORM_PROTOTYPE && pb->q_batch_stride != 0)
        return fail(SA_ERR_UNSUPPORTED, "prototype axis with per-user prototypes is not supported");
    if (pl.proto1 && lse_out) {
        // the one-pass kernel writes the normalisers of the rows it visits;
        // rows outside every user get -inf here first
        e = sa::launch_fill_lse(lse_out, pl.buf_rows * (int64_t)pb->H, status, stream);
        if (e != hipSuccess) return hip_fail(e, "row normaliser fill");
    }
    if (pb->norm == SA_NORM_PROTOTYPE && !pl.proto1) {
        sa::TokLseArgs t{};
        t.users = users;
        t.total_rows = pl.buf_rows;
        t.mask = mask;
        t.P = P;
        t.K = K;
        t.k_stride = pb->k_row_stride ? pb->k_row_stride : hd;
        t.H = pb->H;
        t.m = pb->m;
        t.dh = pb->dh;
        t.c = scale * sa::kLog2e;
        t.lse2_tok = lse2_tok;
        t.lse_out = lse_out;
        t.status = status;
        e = pl.f32 ? sa::launch_f32_tok_lse(t, stream) : sa::launch_bf16_tok_lse(t, stream);
        if (e != hipSuccess) return hip_fail(e, "row normaliser");
    }

    sa::FwdArgs a{};
    a.users = users;
    a.mask = mask;
    a.P = P;
    a.q_batch_stride = pb->q_batch_stride;
    a.K = K;
    a.V = V;
    a.k_stride = pb->k_row_stride ? pb->k_row_stride : hd;
    a.v_stride = pb->v_row_stride ? pb->v_row_stride : hd;
    a.H = pb->H;
    a.m = pb->m;
    a.dh = pb->dh;
    a.c = scale * sa::kLog2e;
    a.G = pl.G;
    a.R_fixed = pl.R_fixed;
    a.R_min = pl.R_min;
    a.split = pl.split;
    a.part = part;
    a.lse2_tok = lse2_tok;
    a.norm = pb->norm;
    a.status = status;
    // a requested per-prototype lse keeps any rounding of the scaled
    // prototypes (the shift cancels in the weights, not in the normaliser), so
    // the streaming kernels then scale unrounded products; a unit scale
    // (the folded production shape) pre-scales exactly
    a.exact_scale = pb->norm == SA_NORM_HISTORY && lse_out != nullptr && a.c != 1.0f;
    if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");
    if (pl.f32) e = sa::launch_f32_forward(a, stream);
    else if (pl.proto1) e = sa::launch_proto_stream(a, lse_out, pl.scfg, stream);
    else if (pl.d128) e = sa::launch_stream_d128(a, pl.scfg, stream);
    else if (pl.stream) e = sa::launch_bf16_stream(a, pl.scfg, stream);
    else e = sa::launch_bf16_forward(a, pl.cfg, stream);
    if (e != hipSuccess) return hip_fail(e, "forward");
    if (ev.stop && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return hip_fail(e, "timing event");

    sa::MergeArgs mg{};
    mg.users = users;
    mg.H = pb->H;
    mg.m = pb->m;
    mg.dh = pb->dh;
    mg.G = pl.G;
    mg.R_fixed = pl.R_fixed;
    mg.R_min = pl.R_min;
    mg.split = pl.split;
    mg.part = part;
    mg.S = S_out;
    mg.lse = pb->norm == SA_NORM_HISTORY ? lse_out : nullptr;
    mg.norm = pb->norm;
    mg.lane_major = !pl.f32;   // the MFMA kernels store their accumulators lane-major
    mg.status = status;
    e = sa::launch_merge(mg, stream);
    if (e != hipSuccess) return hip_fail(e, "merge");
    return SA_OK;
}

sa_status sa_forward_fused_proj(const sa_problem* pb, const void* X, int32_t d_model, const void* Wk, const void* Wv,
                                const void* P, const int32_t* cu_offsets, const uint8_t* mask, float* S_out,
                                float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    const Events ev = take_events();
    clear_stale_error();
    Plan pl;
    sa_status st = make_fused_plan(pb, d_model, &pl);
    if (st != SA_OK) return st;
    if (!cu_offsets) return fail(SA_ERR_INVALID_ARG, "the fused entry takes packed rows: cu_offsets must be non-NULL");
    if (pb->B == 0) return SA_OK;
    if (!X || !Wk || !P || !S_out) return fail(SA_ERR_INVALID_ARG, "X, Wk, P and S_out must be non-NULL");
    if (!Wv && (int64_t)pb->H * pb->dh != d_model)
        return fail(SA_ERR_INVALID_ARG, "Wv == NULL (V = X) needs H*dh == d_model (got %d*%d vs %d)", pb->H, pb->dh,
                    d_model);
    if (!aligned(X, 16) || !aligned(Wk, 16) || (Wv && !aligned(Wv, 16)) || !aligned(P, 16))
        return fail(SA_ERR_INVALID_ARG, "X, Wk, Wv and P must be 16-byte aligned");
    if (!aligned(S_out, 16) || !aligned(lse_out, 4)) return fail(SA_ERR_INVALID_ARG, "misaligned pointer");
    if (pl.total > 0 && (!workspace || workspace_bytes < pl.total))
        return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", pl.total, workspace_bytes);
    if (workspace && !aligned(workspace, kAlign)) return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    unsigned char* ws = (unsigned char*)workspace;
    if (pl.fold_keys) {
        if (Wv) return fail(SA_ERR_UNSUPPORTED, "fused projection, one head of width d_model: V = X only (Wv must be NULL)");
        // scores P (X W_K)^T = (P W_K^T) X^T: the prototypes, scaled by
        // scale * log2(e) and rounded to bf16 once, then the streaming forward
        // over K = V = X with a unit scale (its prototypes are already scaled)
        static_assert((1.0f / sa::kLog2e) * sa::kLog2e == 1.0f, "the unit scale is exact");
        const float scale = pb->scale > 0.f ? pb->scale : 1.0f / sqrtf((float)pb->dh);
        sa::bf16* pf = (sa::bf16*)(ws + pl.off_pfold);
        hipError_t e;
        if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");
        if ((e = sa::launch_fold_keys((const sa::bf16*)P, (const sa::bf16*)Wk, pb->H, pb->m, pb->dh, d_model,
                                      scale * sa::kLog2e, pf, stream)) != hipSuccess)
            return hip_fail(e, "prototype fold");
        sa_problem fp = *pb;
        fp.k_row_stride = d_model;
        fp.v_row_stride = d_model;
        fp.scale = 1.0f / sa::kLog2e;
        g_ev_stop = ev.stop;             // stop after the streaming pass (start is above)
        return sa_forward(&fp, pf, X, X, cu_offsets, nullptr, mask, S_out, lse_out, workspace, pl.fwd_total, stream);
    }
    if (pl.two_pass) {
        if (Wv) return fail(SA_ERR_UNSUPPORTED, "fused projection, two-pass shapes: V = X only (Wv must be NULL)");
        const int hd = pb->H * pb->dh;
        sa::bf16* kbuf = (sa::bf16*)(ws + pl.off_kproj);
        sa::bf16* wt = (sa::bf16*)(ws + pl.off_wt);
        hipError_t e;
        if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");
        sa::TransposeArgs ta{};
        ta.mat[ta.n++] = {(const sa::bf16*)Wk, wt, d_model, hd};
        if ((e = sa::launch_transpose(ta, stream)) != hipSuccess) return hip_fail(e, "weight transpose");
        sa::ProjectArgs pa{};
        pa.X = (const sa::bf16*)X;
        pa.x_stride = d_model;
        pa.wt = wt;
        pa.out = kbuf;
        pa.rows = pl.buf_rows;
        if ((e = sa::launch_project(pa, d_model, hd, device_info().cus, stream)) != hipSuccess)
            return hip_fail(e, "key projection");
        sa_problem fp = *pb;
        fp.k_row_stride = hd;
        fp.v_row_stride = d_model;
        g_ev_stop = ev.stop;             // stop after the streaming pass (start is above)
        return sa_forward(&fp, P, kbuf, X, cu_offsets, nullptr, mask, S_out, lse_out, workspace, pl.fwd_total, stream);
    }
    sa::Users users{};
    users.cu = cu_offsets;
    users.B = pb->B;
    const float scale = pb->scale > 0.f ? pb->scale : 1.0f / sqrtf((float)pb->dh);
    sa::Partials part{(float*)(ws + pl.off_acc), (float*)(ws + pl.off_M), (float*)(ws + pl.off_Z)};

    sa::FusedArgs a{};
    a.users = users;
    a.mask = mask;
    a.X = X;
    a.Wk = Wk;
    a.Wv = Wv;
    a.P = P;
    a.q_batch_stride = pb->q_batch_stride;
    a.H = pb->H;
    a.m = pb->m;
    a.d_model = d_model;
    a.c = scale * sa::kLog2e;
    a.G = pl.G;
    a.R_fixed = pl.R_fixed;
    a.R_min = pl.R_min;
    a.part = part;
    hipError_t e;
    const int32_t* status = nullptr;
    if (pl.check_offsets) {
        int32_t* sw = (int32_t*)(ws + pl.off_status);
        if ((e = sa::launch_check_offsets(cu_offsets, pb->B, pb->total_rows, sw, stream)) != hipSuccess)
            return hip_fail(e, "offsets check");
        status = sw;
    }
    a.status = status;
    if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");
    e = sa::launch_fused(a, stream);
    if (e != hipSuccess) return hip_fail(e, "fused forward");
    if (ev.stop && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return hip_fail(e, "timing event");

    sa::MergeArgs mg{};
    mg.users = users;
    mg.H = pb->H;
    mg.m = pb->m;
    mg.dh = pb->dh;
    mg.G = pl.G;
    mg.R_fixed = pl.R_fixed;
    mg.R_min = pl.R_min;
    mg.split = pl.split;
    mg.part = part;
    mg.S = S_out;
    mg.lse = lse_out;
    mg.norm = SA_NORM_HISTORY;
    mg.lane_major = 1;
    mg.status = status;
    e = sa::launch_merge(mg, stream);
    if (e != hipSuccess) return hip_fail(e, "merge");
    return SA_OK;
}

size_t sa_forward_fused_proj_workspace_size(const sa_problem* pb, int32_t d_model) {
    Plan pl;
    if (!pb || make_fused_plan(pb, d_model, &pl) != SA_OK) return 0;
    return pl.total;
}

}  // extern "C"

namespace {

// Workspace of the STCA attention: W_Q and W_V transposed to [out][in], the
// block table, the queries q = x W_Q [T][D] and alpha X [T][h][D] (bf16).
struct StcaPlan {
    size_t off_wqt = 0, off_wvt = 0, off_table = 0, off_q = 0, off_y = 0, total = 0;
    int grid = 0, dh = 0;
    int64_t x_stride = 0;
    float c = 0.f;
};

sa_status make_stca_plan(const sa_stca_problem* pb, StcaPlan* sp) {
    if (!pb) return fail(SA_ERR_INVALID_ARG, "problem is NULL");
    if (pb->flags != 0) return fail(SA_ERR_INVALID_ARG, "flags must be 0");
    if (pb->B < 0 || pb->T < 0 || pb->total_rows < 0)
        return fail(SA_ERR_INVALID_ARG, "B, T and total_rows must be >= 0 (got %d, %d, %lld)", pb->B, pb->T,
                    (long long)pb->total_rows);
    if (pb->D <= 0 || pb->h <= 0 || pb->D % pb->h != 0)
        return fail(SA_ERR_INVALID_ARG, "D and h must be positive with h dividing D (got D=%d h=%d)", pb->D, pb->h);
    const int dh = pb->D / pb->h;
    if (pb->h % 2 != 0 || !sa::stca_supported(pb->D, dh))
        return fail(SA_ERR_UNSUPPORTED, "STCA attention: D == 1024 with dh in {64, 128} (got D=%d h=%d)", pb->D,
                    pb->h);
    const int64_t xs = pb->x_row_stride == 0 ? pb->D : pb->x_row_stride;
    if (xs < pb->D || xs % 8 != 0)
        return fail(SA_ERR_INVALID_ARG, "x_row_stride must be 0 or a multiple of 8 that is >= D (got %lld)",
                    (long long)pb->x_row_stride);
    if (!isfinite(pb->scale) || pb->scale < 0.f) return fail(SA_ERR_INVALID_ARG, "scale must be finite and >= 0");
    const int64_t chunks = ((int64_t)pb->T + sa::kStcaTargets - 1) / sa::kStcaTargets + pb->B;
    const int64_t grid = (chunks * (pb->h / 2) + 7) / 8 * 8;
    if (grid > (int64_t)1 << 30) return fail(SA_ERR_UNSUPPORTED, "too many targets and users for one launch");
    sp->grid = (int)std::max<int64_t>(grid, 8);
    sp->dh = dh;
    sp->x_stride = xs;
    sp->c = (pb->scale == 0.f ? 1.f / sqrtf((float)dh) : pb->scale) * sa::kLog2e;
    const size_t dd = (size_t)pb->D * pb->D;
    size_t off = 0;
    sp->off_wqt = off;
    off = align_up(off + 2 * dd);
    sp->off_wvt = off;
    off = align_up(off + 2 * dd);
    sp->off_table = off;
    off = align_up(off + 32 * (size_t)sp->grid);
    sp->off_q = off;
    off = align_up(off + 2 * (size_t)pb->T * pb->D);
    sp->off_y = off;
    off = align_up(off + 2 * (size_t)pb->T * pb->h * pb->D);
    sp->total = off;
    return SA_OK;
}

}  // namespace

extern "C" {

sa_status sa_stca_attention(const sa_stca_problem* pb, const void* xt, const void* X, const void* Wq, const void* Wk,
                            const void* Wv, const int32_t* cu_offsets, const int32_t* t_offsets,
                            const int32_t* windows, float* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    g_err[0] = 0;
    const Events ev = take_events();
    clear_stale_error();
    StcaPlan sp;
    sa_status st = make_stca_plan(pb, &sp);
    if (st != SA_OK) return st;
    if (pb->T == 0) return SA_OK;
    if (!xt || !Wq || !Wk || !Wv || !t_offsets || !out)
        return fail(SA_ERR_INVALID_ARG, "xt, Wq, Wk, Wv, t_offsets and out must be non-NULL");
    if (pb->B > 0 && (!cu_offsets || (!X && pb->total_rows > 0)))
        return fail(SA_ERR_INVALID_ARG, "cu_offsets (and X when total_rows > 0) must be non-NULL");
    if (!aligned(xt, 16) || !aligned(X, 16) || !aligned(Wq, 16) || !aligned(Wk, 16) || !aligned(Wv, 16) ||
        !aligned(out, 16) || !aligned(windows, 4) || !aligned(cu_offsets, 4) || !aligned(t_offsets, 4))
        return fail(SA_ERR_INVALID_ARG, "xt, X, Wq, Wk, Wv and out must be 16-byte aligned");
    if (!workspace || workspace_bytes < sp.total)
        return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", sp.total, workspace_bytes);
    if (!aligned(workspace, kAlign)) return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    unsigned char* ws = (unsigned char*)workspace;
    const sa::bf16* wqt = (const sa::bf16*)(ws + sp.off_wqt);
    const sa::bf16* wvt = (const sa::bf16*)(ws + sp.off_wvt);
    sa::bf16* q = (sa::bf16*)(ws + sp.off_q);
    sa::bf16* y = (sa::bf16*)(ws + sp.off_y);
    const int D = pb->D, h = pb->h, dh = sp.dh, T = pb->T;
    sa::StcaArgs a{};
    a.X = (const sa::bf16*)X;
    a.x_stride = sp.x_stride;
    a.qm = q;
    a.wk = (const sa::bf16*)Wk;
    a.cu = cu_offsets;
    a.tcu = t_offsets;
    a.win = windows;
    a.y = y;
    a.table = (int4*)(ws + sp.off_table);
    a.B = pb->B;
    a.T = T;
    a.h = h;
    a.D = D;
    a.grid = sp.grid;
    a.c = sp.c;

    hipError_t e;
    sa::TransposeArgs ta{};
    ta.mat[ta.n++] = {(const sa::bf16*)Wq, (sa::bf16*)wqt, D, D};
    ta.mat[ta.n++] = {(const sa::bf16*)Wv, (sa::bf16*)wvt, D, D};
    if ((e = sa::launch_transpose(ta, stream)) != hipSuccess) return hip_fail(e, "weight transpose");
    if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");
    // q = x W_Q for every target
    sa::GemmArgs g1{};
    g1.A = (const sa::bf16*)xt;
    g1.Bt = wqt;
    g1.C = q;
    g1.lda = g1.ldb = g1.ldc = D;
    g1.M = T;
    g1.N = D;
    g1.K = D;
    g1.batch = 1;
    if ((e = sa::launch_gemm_nt(g1, true, stream)) != hipSuccess) return hip_fail(e, "query projection");
    if ((e = sa::launch_stca(a, dh, stream)) != hipSuccess) return hip_fail(e, "STCA attention");
    // out[:, head block] = (alpha X)[:, head] W_V[:, head block], per head
    sa::GemmArgs g3{};
    g3.A = y;
    g3.lda = (int64_t)h * D;
    g3.sA = D;
    g3.Bt = wvt;
    g3.ldb = D;
    g3.sB = (int64_t)dh * D;
    g3.C = out;
    g3.ldc = D;
    g3.sC = dh;
    g3.M = T;
    g3.N = dh;
    g3.K = D;
    g3.batch = h;
    if ((e = sa::launch_gemm_nt(g3, false, stream)) != hipSuccess) return hip_fail(e, "output projection");
    if (ev.stop && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return hip_fail(e, "timing event");
    return SA_OK;
}

size_t sa_stca_workspace_size(const sa_stca_problem* pb) {
    StcaPlan sp;
    return make_stca_plan(pb, &sp) == SA_OK ? sp.total : 0;
}

}  // extern "C"

namespace {

constexpr int kMaxRefineLayers = 8;

// Workspace of the refinement: the attention pass's own workspace, then the
// attention output, the per-user and first-layer queries, and the weights
// transposed to [out][in] (Wq, W1, W3, W2 per layer).
struct RefinePlan {
    Plan att;
    size_t off_xhat = 0, off_q = 0, off_q0 = 0, off_w = 0, total = 0;
};

sa_status make_refine_plan(const sa_problem* pb, int32_t d_model, int32_t n_layers, RefinePlan* rp) {
    if (!pb) return fail(SA_ERR_INVALID_ARG, "problem is NULL");
    if (pb->flags != 0) return fail(SA_ERR_INVALID_ARG, "refinement: flags must be 0");
    if (pb->q_batch_stride != 0 || pb->L_max != 0 || pb->k_row_stride != 0 || pb->v_row_stride != 0)
        return fail(SA_ERR_INVALID_ARG, "refinement: q_batch_stride, L_max and the row strides must be 0");
    if (n_layers < 1 || n_layers > kMaxRefineLayers)
        return fail(SA_ERR_INVALID_ARG, "n_layers must be in 1..%d (got %d)", kMaxRefineLayers, n_layers);
    if ((int64_t)pb->H * pb->dh != d_model)
        return fail(SA_ERR_INVALID_ARG, "refinement aggregates X itself: needs H*dh == d_model (got %d*%d vs %d)",
                    pb->H, pb->dh, d_model);
    sa_status st = make_fused_plan(pb, d_model, &rp->att);
    if (st != SA_OK) return st;
    if (rp->att.two_pass || !sa::fused_supported(d_model, pb->m, pb->dh))
        return fail(SA_ERR_UNSUPPORTED, "refinement: dh == 32, d_model in {128, 256}, m in {64, 128, 256} "
                                        "(got dh=%d d_model=%d m=%d)", pb->dh, d_model, pb->m);
    if (!sa::sketch_supported(d_model))
        return fail(SA_ERR_UNSUPPORTED, "refinement: d_model must be 128 or 256 (got %d)", d_model);
    const size_t bhmd = (size_t)pb->B * pb->H * pb->m * pb->dh, d = (size_t)d_model;
    size_t off = align_up(rp->att.total);
    rp->off_xhat = off;
    off = align_up(off + sizeof(float) * bhmd);
    rp->off_q = off;
    off = align_up(off + 2 * bhmd);
    rp->off_q0 = off;
    off = align_up(off + 2 * (size_t)pb->H * pb->m * pb->dh);
    rp->off_w = off;
    off = align_up(off + 2 * 7 * d * d * (size_t)n_layers);
    rp->total = off;
    return SA_OK;
}

}  // namespace

extern "C" {

sa_status sa_refine_forward(const sa_problem* pb, const void* X, int32_t d_model, const float* P0, int32_t n_layers,
                            const sa_refine_layer* layers, float eps, const int32_t* cu_offsets, const uint8_t* mask,
                            float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    const Events ev = take_events();
    clear_stale_error();
    RefinePlan rp;
    sa_status st = make_refine_plan(pb, d_model, n_layers, &rp);
    if (st != SA_OK) return st;
    if (!cu_offsets) return fail(SA_ERR_INVALID_ARG, "refinement takes packed rows: cu_offsets must be non-NULL");
    if (!layers) return fail(SA_ERR_INVALID_ARG, "layers is NULL");
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(SA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    for (int l = 0; l < n_layers; ++l) {
        const sa_refine_layer& L = layers[l];
        const void* ptrs[] = {L.Wq, L.Wk, L.ln1_g, L.ln1_b, L.W1, L.W3, L.W2, L.ln2_g, L.ln2_b};
        for (const void* q : ptrs)
            if (!q) return fail(SA_ERR_INVALID_ARG, "layer %d: every weight pointer must be non-NULL", l);
        if (!aligned(L.Wq, 16) || !aligned(L.Wk, 16) || !aligned(L.W1, 16) || !aligned(L.W3, 16) ||
            !aligned(L.W2, 16) || !aligned(L.ln1_g, 4) || !aligned(L.ln1_b, 4) || !aligned(L.ln2_g, 4) ||
            !aligned(L.ln2_b, 4))
            return fail(SA_ERR_INVALID_ARG, "layer %d: matrices must be 16-byte aligned", l);
    }
    if (pb->B == 0) return SA_OK;
    if (!X || !P0 || !out) return fail(SA_ERR_INVALID_ARG, "X, P0 and out must be non-NULL");
    if (!aligned(X, 16) || !aligned(P0, 16) || !aligned(out, 16))
        return fail(SA_ERR_INVALID_ARG, "X, P0 and out must be 16-byte aligned");
    if (!workspace || workspace_bytes < rp.total)
        return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", rp.total, workspace_bytes);
    if (!aligned(workspace, kAlign)) return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    unsigned char* ws = (unsigned char*)workspace;
    float* xhat = (float*)(ws + rp.off_xhat);
    sa::bf16* q = (sa::bf16*)(ws + rp.off_q);
    sa::bf16* q0 = (sa::bf16*)(ws + rp.off_q0);
    sa::bf16* wt = (sa::bf16*)(ws + rp.off_w);
    const int D = d_model;
    const size_t dd = (size_t)D * D;
    auto wq_t = [&](int l) { return wt + 7 * dd * l; };
    auto w1_t = [&](int l) { return wt + 7 * dd * l + dd; };
    auto w3_t = [&](int l) { return wt + 7 * dd * l + 3 * dd; };
    auto w2_t = [&](int l) { return wt + 7 * dd * l + 5 * dd; };

    hipError_t e;
    if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");

    // weights to [out][in]
    sa::TransposeArgs ta{};
    for (int l = 0; l < n_layers; ++l) {
        ta.mat[ta.n++] = {(const sa::bf16*)layers[l].Wq, wq_t(l), D, D};
        ta.mat[ta.n++] = {(const sa::bf16*)layers[l].W1, w1_t(l), D, 2 * D};
        ta.mat[ta.n++] = {(const sa::bf16*)layers[l].W3, w3_t(l), D, 2 * D};
        ta.mat[ta.n++] = {(const sa::bf16*)layers[l].W2, w2_t(l), 2 * D, D};
    }
    if ((e = sa::launch_transpose(ta, stream)) != hipSuccess) return hip_fail(e, "weight transpose");

    // first-layer queries P0 Wq_0 (shared by every user)
    sa::SketchArgs sk{};
    sk.m = pb->m;
    sk.H = pb->H;
    sk.dh = pb->dh;
    sk.eps = eps;
    sk.mode = 1;
    sk.rows = pb->m;
    sk.base = P0;
    sk.wqt = wq_t(0);
    sk.q = q0;
    if ((e = sa::launch_sketch(sk, D, stream)) != hipSuccess) return hip_fail(e, "query projection");

    for (int l = 0; l < n_layers; ++l) {
        sa_problem pl = *pb;
        pl.q_batch_stride = l == 0 ? 0 : (int64_t)pb->H * pb->m * pb->dh;
        st = sa_forward_fused_proj(&pl, X, d_model, layers[l].Wk, nullptr, l == 0 ? (const void*)q0 : (const void*)q,
                                   cu_offsets, mask, xhat, nullptr, workspace, rp.att.total, stream);
        if (st != SA_OK) return st;
        sa::SketchArgs u = sk;
        u.mode = 0;
        u.rows = pb->B * pb->m;
        u.base = l == 0 ? P0 : out;
        u.base_shared = l == 0;
        u.xhat = xhat;
        u.ln1_g = layers[l].ln1_g;
        u.ln1_b = layers[l].ln1_b;
        u.ln2_g = layers[l].ln2_g;
        u.ln2_b = layers[l].ln2_b;
        u.w1t = w1_t(l);
        u.w3t = w3_t(l);
        u.w2t = w2_t(l);
        u.wqt = l + 1 < n_layers ? wq_t(l + 1) : nullptr;
        u.q = q;
        u.out = out;
        if ((e = sa::launch_sketch(u, D, stream)) != hipSuccess) return hip_fail(e, "sketch update");
    }
    if (ev.stop && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return hip_fail(e, "timing event");
    return SA_OK;
}

}  // extern "C"

namespace {

// Backward plan: the forward's validation, the kernels' own limits and work
// split, and the workspace (dense prefix, D, lse2, dS in bf16, dP partials).
struct BwdPlan {
    Plan fw;
    int G = 1, G1 = 1;
    size_t off_vcu = 0, off_D = 0, off_L2 = 0, off_dsb = 0, off_part = 0, total = 0;
};

sa_status make_bwd_plan(const sa_problem* pb_in, bool packed, BwdPlan* bp) {
    if (!pb_in) return fail(SA_ERR_INVALID_ARG, "problem is NULL");
    if (pb_in->flags & ~SA_FLAG_BF16_GRADS)
        return fail(SA_ERR_INVALID_ARG, "backward: flags must be 0 or SA_FLAG_BF16_GRADS (got %d)", pb_in->flags);
    sa_problem q = *pb_in;      // the forward's checks see flags = 0
    q.flags = 0;
    const sa_problem* pb = &q;
    sa_status st = make_plan(pb, packed, &bp->fw, 0);
    if (st != SA_OK) return st;
    if (pb->dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "backward: bf16 inputs only");
    if (pb->norm != SA_NORM_HISTORY) return fail(SA_ERR_UNSUPPORTED, "backward: history axis only");
    if (!sa::bwd_supported(pb->dh, pb->m))
        return fail(SA_ERR_UNSUPPORTED, "backward: dh in {32, 64} and m in {32, 64, 128, 256} (got dh=%d m=%d)", pb->dh,
                    pb->m);
    const int cus = device_info().cus;
    int NH, PB;
    sa::bwd_dp_shape(pb->m, pb->H, &NH, &PB);
    const int groups = (pb->H + NH - 1) / NH;
    const int64_t rows_upper = pb->L_max > 0 ? (int64_t)pb->B * pb->L_max : pb->total_rows;
    if (pb->chunk_rows > 0) {
        const int64_t G = (rows_upper + pb->chunk_rows - 1) / pb->chunk_rows;
        bp->G = bp->G1 = (int)(G > 0 ? G : 1);
    } else {
        // dP pass: blocks of 8 waves; at dh = 64 the ring kernel holds ~150
        // registers, so one block fits a CU (a grid of two per CU ran in two
        // rounds: the backward 0.5-0.9 % slower, the dP merge 37 against 20 us
        // for twice the partials); at dh = 32 (~110 registers) two fit
        const int dp_bpc = pb->dh == 64 ? 1 : 2;
        bp->G = cus * dp_bpc / groups > 0 ? cus * dp_bpc / groups : 1;
        int bpc = kDkdvBlocksPerCu;
        if (pb->dh == 64 && !(pb_in->flags & SA_FLAG_BF16_GRADS)) bpc = kDkdvBlocksPerCuF32d64;
        if (g_tune.bwd_blocks_per_cu > 0) bpc = g_tune.bwd_blocks_per_cu;
        bp->G1 = cus * bpc / pb->H > 0 ? cus * bpc / pb->H : 1;
    }
    const size_t bhm = (size_t)pb->B * pb->H * pb->m;
    size_t off = 0;
    bp->off_vcu = off;
    off = align_up(off + sizeof(int32_t) * ((size_t)pb->B + 1));
    bp->off_D = off;
    off = align_up(off + sizeof(float) * bhm);
    bp->off_L2 = off;
    off = align_up(off + sizeof(float) * bhm);
    bp->off_dsb = off;
    off = align_up(off + 2 * bhm * pb->dh);
    bp->off_part = off;
    off = align_up(off + sizeof(float) * ((size_t)bp->G + pb->B) * pb->H * pb->m * pb->dh);
    bp->total = off;
    return SA_OK;
}

}  // namespace

extern "C" {

sa_status sa_backward(const sa_problem* pb, const void* P, const void* K, const void* V, const int32_t* cu_offsets,
                      const int32_t* lengths, const uint8_t* mask, const float* S, const float* lse, const float* dS,
                      float* dP, void* dK, void* dV, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    const Events ev = take_events();
    clear_stale_error();
    BwdPlan bp;
    const bool packed = cu_offsets != nullptr;
    sa_status st = make_bwd_plan(pb, packed, &bp);
    if (st != SA_OK) return st;
    if (lengths && packed) return fail(SA_ERR_INVALID_ARG, "lengths is only valid for the dense layout");
    if (pb->B == 0) return SA_OK;
    if (!P || !K || !V || !S || !lse || !dS || !dP || !dK || !dV)
        return fail(SA_ERR_INVALID_ARG, "P, K, V, S, lse, dS, dP, dK and dV must be non-NULL");
    if (!aligned(P, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(S, 16) || !aligned(dS, 16) ||
        !aligned(dP, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(lse, 4))
        return fail(SA_ERR_INVALID_ARG, "P, K, V, S, dS, dP, dK and dV must be 16-byte aligned");
    if (!workspace || workspace_bytes < bp.total)
        return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", bp.total, workspace_bytes);
    if (!aligned(workspace, kAlign)) return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    unsigned char* ws = (unsigned char*)workspace;
    sa::Users users{};
    users.cu = cu_offsets;
    users.B = pb->B;
    users.L_max = pb->L_max;
    hipError_t e;
    if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return hip_fail(e, "timing event");
    if (!packed && lengths) {
        users.vcu = (int32_t*)(ws + bp.off_vcu);
        e = sa::launch_dense_vcu(lengths, pb->B, pb->L_max, (int32_t*)(ws + bp.off_vcu), stream);
        if (e != hipSuccess) return hip_fail(e, "dense offsets");
    }
    const int64_t hd = (int64_t)pb->H * pb->dh;
    const float scale = pb->scale > 0.f ? pb->scale : 1.0f / sqrtf((float)pb->dh);
    sa::BwdArgs a{};
    a.users = users;
    a.mask = mask;
    a.P = P;
    a.q_batch_stride = pb->q_batch_stride;
    a.K = K;
    a.V = V;
    a.k_stride = pb->k_row_stride ? pb->k_row_stride : hd;
    a.v_stride = pb->v_row_stride ? pb->v_row_stride : hd;
    a.H = pb->H;
    a.m = pb->m;
    a.dh = pb->dh;
    a.c = scale;
    a.c2 = scale * sa::kLog2e;
    a.G = bp.G;
    a.G1 = bp.G1;
    a.R_fixed = pb->chunk_rows;
    a.R_min = sa::kRowAlign;
    a.S = S;
    a.lse = lse;
    a.dS = dS;
    a.Dv = (float*)(ws + bp.off_D);
    a.L2v = (float*)(ws + bp.off_L2);
    a.dSb = (sa::bf16*)(ws + bp.off_dsb);
    a.dK = dK;
    a.dV = dV;
    a.grads_bf16 = (pb->flags & SA_FLAG_BF16_GRADS) != 0;
    a.part = sa::Partials{(float*)(ws + bp.off_part), nullptr, nullptr};
    a.dP = dP;
    a.per_user = pb->q_batch_stride != 0;
    a.dp_register_staged = g_tune.bwd_dp_register_staged != 0;
    if ((e = sa::launch_backward(a, stream)) != hipSuccess) return hip_fail(e, "backward");
    if (ev.stop && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return hip_fail(e, "timing event");
    return SA_OK;
}

size_t sa_backward_workspace_size(const sa_problem* pb) {
    BwdPlan bp;
    if (!pb || make_bwd_plan(pb, pb->L_max == 0, &bp) != SA_OK) return 0;
    return bp.total;
}

size_t sa_refine_workspace_size(const sa_problem* pb, int32_t d_model, int32_t n_layers) {
    RefinePlan rp;
    if (make_refine_plan(pb, d_model, n_layers, &rp) != SA_OK) return 0;
    return rp.total;
}

sa_status sa_set_timing_events(hipEvent_t start, hipEvent_t stop) {
    if ((start == nullptr) != (stop == nullptr)) return fail(SA_ERR_INVALID_ARG, "give both timing events or neither");
    g_ev_start = start;
    g_ev_stop = stop;
    return SA_OK;
}

sa_status sa_set_tuning(const sa_tuning* t) {
    if (!t) {
        g_tune = sa_tuning{};
        return SA_OK;
    }
    if (t->register_staged < 0 || t->register_staged > 1 || t->bwd_dp_register_staged < 0 ||
        t->bwd_dp_register_staged > 1)
        return fail(SA_ERR_INVALID_ARG, "register_staged flags must be 0 or 1");
    if (!(t->stream_waves == 0 || t->stream_waves == 8 || t->stream_waves == 16))
        return fail(SA_ERR_INVALID_ARG, "stream_waves must be 0, 8 or 16 (got %d)", t->stream_waves);
    if (t->blocks_per_cu < 0 || t->blocks_per_cu > 64 || t->bwd_blocks_per_cu < 0 || t->bwd_blocks_per_cu > 64)
        return fail(SA_ERR_INVALID_ARG, "blocks per CU must be in 0..64");
    if (t->range_split < 0 || t->range_split > 99)
        return fail(SA_ERR_INVALID_ARG, "range_split must be in 0..99 (got %d)", t->range_split);
    if (!(t->bf16_tile_mb == 0 || t->bf16_tile_mb == 16 || t->bf16_tile_mb == 32 || t->bf16_tile_mb == 64) ||
        !(t->bf16_tile_nw == 0 || t->bf16_tile_nw == 4 || t->bf16_tile_nw == 8) ||
        ((t->bf16_tile_mb == 0) != (t->bf16_tile_nw == 0)))
        return fail(SA_ERR_INVALID_ARG, "bf16 tile: mb in {16, 32, 64} and nw in {4, 8}, or both 0");
    g_tune = *t;
    return SA_OK;
}

int32_t sa_check_offsets_host(const int32_t* cu, int32_t B, int64_t total_rows, int32_t* first_bad) {
    int32_t bits = 0, first = -1;
    if (cu && B >= 0) {
        for (int32_t b = 0; b <= B; ++b) {
            const int32_t x = sa::offsets_entry_bits(cu, b, B, total_rows);
            if (x && first < 0) first = b;
            bits |= x;
        }
    }
    if (first_bad) *first_bad = first;
    return bits;
}

const char* sa_status_string(int32_t status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARG: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported problem";
        case SA_ERR_WORKSPACE: return "workspace too small";
        case SA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* sa_last_error(void) { return g_err; }

int sa_version(void) { return SA_VERSION_MAJOR * 10000 + SA_VERSION_MINOR * 100 + SA_VERSION_PATCH; }

}  // extern "C"

// ---------------------------------------------------------------------------
// sa_forward_noalloc: sa_forward with a workspace the library holds itself,
// for callers that cannot allocate device memory.  The workspace is a
// file-scope device array; every device the library runs on holds its own
// copy from the first call until the process ends.  In host code the array's
// name is only a stand-in for the symbol, never a device address: the address
// of a device's copy comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is handed to kernels.

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;   // 64 MiB per device

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device (nullptr on failure,
// with the error text set).
void* scratch_on_current_device() {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        fail(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        fail(SA_ERR_HIP, "device %d is beyond the %d devices this entry point serves", dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

extern "C" {

size_t sa_forward_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

sa_status sa_forward_noalloc(const sa_problem* pb, const void* P, const void* K, const void* V,
                             const int32_t* cu_offsets, const int32_t* lengths, const uint8_t* mask, float* S_out,
                             float* lse_out, hipStream_t stream) {
    g_err[0] = 0;
    Plan pl;
    sa_status st = make_plan(pb, cu_offsets != nullptr, &pl);
    if (st != SA_OK) {
        take_events();
        return st;
    }
    if (pl.total > kNoAllocScratchBytes) {
        take_events();
        return fail(SA_ERR_WORKSPACE,
                    "this problem needs %zu bytes of workspace; sa_forward_noalloc holds %zu (use sa_forward with a "
                    "caller-allocated workspace)", pl.total, kNoAllocScratchBytes);
    }
    void* ws = nullptr;
    if (pb->B > 0 && pl.total > 0) {
        ws = scratch_on_current_device();
        if (!ws) {
            take_events();
            return SA_ERR_HIP;
        }
    }
    return sa_forward(pb, P, K, V, cu_offsets, lengths, mask, S_out, lse_out, ws, ws ? kNoAllocScratchBytes : 0,
                      stream);
}

}  // extern "C"
