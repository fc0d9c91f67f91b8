// sa_stca.hip -- STCA single-query target-to-history cross attention with the
// reordering of appendix G.2.1 of the SequenceO1 paper:
//     q = x W_Q,  u_h = q_h W_K[:, h]^T,  alpha = softmax(u_h X^T / sqrt(dh)),
//     o_h = (alpha X) W_V[:, h]
// for every target of every user of a packed batch; a user's targets share
// its history rows (the multi-request batching of section 4.2).  The host
// sequence (sa_api.hip) is: q = x W_Q for all targets (sa_gemm.hip), this
// file's setup launch and fused attention kernel, which writes alpha X per
// (target, head), then the per-head products with W_V (sa_gemm.hip).
//
// Attention block = (user, head pair, 16 targets): 32 query columns, one
// 16-column MFMA tile per head.  Eight waves, two per SIMD; wave (cs, hs)
// owns channels [cs D/4, (cs+1) D/4) of the D-wide rows for head 2 hp + hs,
// and the two waves of a channel slice (one SIMD) share its ring:
//   * prologue: u^T over the slice's channels for the wave's head (MFMA with
//     W_K and q), staged through LDS into the score product's B operand,
//     kept in registers;
//   * loop over 32-row tiles of the rows the block's targets see: the slice
//     of every row streams through the slice's two-stage LDS ring by
//     direct-to-LDS loads, half of each stage issued by each of its two
//     waves; partial scores over the slice (MFMA) go to a double-buffered
//     LDS exchange; the tile's one block barrier certifies the next stage
//     (each wave has waited for its own half) and frees the slot the wave
//     pair has read, which is then refilled; every wave adds the other three
//     slices' partials of its head to its own (in slice order) and runs the
//     online softmax on the full scores.  The four slices' sums differ only
//     in rounding, and each wave normalises its channels with its own
//     running sum, so every output slice is a weighted mean under one
//     consistent set of weights.  alpha X over the slice's channels
//     accumulates on MFMA from transposed LDS reads of the same ring stage.
//     The loop is software-pipelined: tile t+1's scores are computed while
//     tile t's weights are formed;
//   * epilogue: alpha X normalised, in bf16, written row by row through LDS.
// (Four waves each with both heads of a slice ran at one wave per SIMD: the
// wave then held twice the accumulators and operands, ~450 VGPRs and AGPRs,
// and its LDS reads, exchange, barrier and MFMAs could not overlap another
// wave's.)
// Ring rows are XOR-swizzled per 16-byte chunk so that the row reads of the
// score product and the transposed reads of the aggregation are both free of
// bank conflicts.  A sa_stca_prep_kernel launch first builds the block table
// from the target offsets on the device (no host reads) and zeroes the rows
// of targets outside every user.
#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kStcaWaves = 4;
// fast-loop range of a lane's tile sum of weights 2^(s c) (maximum fixed at 0)
constexpr float kStcaHiBound = 4294967296.0f;      // 2^32
constexpr float kStcaLoBound = 2.3283064365e-10f;  // 2^-32

typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x4 lds_ld4(uint32_t a) { return *(const lds_f32x4*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st4(uint32_t a, f32x4 v) { *(lds_f32x4*)(uintptr_t)a = v; }
__device__ __forceinline__ bf16x8 lds_ld8(uint32_t a) { return *(const lds_bf16x8*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st_b4(uint32_t a, bf16x4 v) { *(lds_bf16x4*)(uintptr_t)a = v; }

// 16-byte chunk swizzle of a ring row (XOR on the chunk index, a function of
// row % 16), for the 64 four-byte banks of an LDS cycle: the 16 rows read by
// one 16-lane group of the score operand land on 16 distinct chunks of the
// 256-byte bank window, and the 8 rows read by a 32-lane group of the
// transposed reads on 8 distinct 32-byte chunk pairs
__device__ __forceinline__ int stca_swz(int r) { return 2 * (r & 7) + ((r >> 3) & 1); }

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) { return __builtin_convertvector(v, bf16x4); }

}  // namespace

template <int D, int DH>
__global__ __launch_bounds__(2 * kStcaWaves * 64, 2) void sa_stca_kernel(StcaArgs a) {
    constexpr int NW = kStcaWaves;         // channel slices
    constexpr int DW = D / NW;             // channels per slice
    constexpr int KC = DW / 32;            // 32-channel k-steps of the score product
    constexpr int DB = DW / 16;            // 16-channel row blocks of the aggregate
    constexpr int ROWB = DW * 2;           // bytes of a slice of one row
    constexpr int STAGE = 32 * ROWB;       // bytes of one 32-row ring stage
    constexpr int OPS = STAGE / 1024;      // direct-to-LDS ops per stage (both waves of a slice)
    constexpr int OPW = OPS / 2;           // of them per wave
    constexpr int EK = DH / 32;            // k-steps over dh
    static_assert(DW == 256 && DH % 32 == 0 && OPS * 1024 == STAGE && OPW * 2 == OPS,
                  "compiled for 256 channels per slice");

    __shared__ __attribute__((aligned(1024))) unsigned char ring[NW][2][STAGE];
    __shared__ __attribute__((aligned(1024))) f32x4 xchg[2][NW][4][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // wave (cs, hs): channel slice cs of head 2 hp + hs; the two waves of a
    // slice sit on one SIMD and share its ring
    const int cs = wave & (NW - 1), hs = wave / NW;

    // block -> (user, target chunk, head pair): XCD x (blockIdx % 8) takes the
    // x-th contiguous run of the table, so a user's blocks share one L2
    const int G = gridDim.x;
    const int Lb = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    // (everything the block needs before its first loads comes in its two
    // table entries, so they can all be issued after one round trip)
    const int4 ent = a.table[2 * Lb];
    const int b = __builtin_amdgcn_readfirstlane(ent.x);
    if (b < 0) return;
    const int tb = __builtin_amdgcn_readfirstlane(ent.y);
    const int nt = __builtin_amdgcn_readfirstlane(ent.z);
    const int hp = __builtin_amdgcn_readfirstlane(ent.w);
    const int4 ent2 = a.table[2 * Lb + 1];
    const int row0 = __builtin_amdgcn_readfirstlane(ent2.x);   // absolute first row the block streams
    const int nrows = __builtin_amdgcn_readfirstlane(ent2.y);
    const int ntiles = (nrows + 31) / 32;
    const int hh = 2 * hp + hs;            // this wave's head

    // this lane's target (column l16) and its window, relative to the
    // block's first row (needed only once the loop starts)
    const bool tv = l16 < nt;
    const int tl = tb + (tv ? l16 : 0);
    int qlo = 0, qhi = 0;
    if (tv) {
        const int u0 = a.cu[b], nu = a.cu[b + 1] - u0;
        int wlo = 0, whi = nu;
        if (a.win != nullptr) {
            wlo = min(max(a.win[2 * (int64_t)tl], 0), nu);
            whi = max(wlo, min(max(a.win[2 * (int64_t)tl + 1], 0), nu));
        }
        qlo = u0 + wlo - row0;
        qhi = u0 + whi - row0;
    }

    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0][0];
    const uint32_t my_ring = ring_lds + (uint32_t)(cs * 2 * STAGE);
    const uint32_t xch_lds = (uint32_t)(uintptr_t)(lds_void*)&xchg[0][0][0][0];

    // ---- prologue: u^T[d][t] = sum_e W_K[d][hh dh + e] q[t][hh dh + e] over
    // the slice's channels d, this wave's head (q = x W_Q comes precomputed);
    // staged through the slice's ring (as [hs][t][channel], rows swizzled by
    // t; the two heads' waves write disjoint rows) into the score B operand
    bf16x8 uf[KC];
    {
        bf16x8 qb[EK];
#pragma unroll
        for (int ek = 0; ek < EK; ++ek) qb[ek] = *(const bf16x8*)(a.qm + (int64_t)tl * D + hh * DH + 32 * ek + 8 * g);
        // W_K operands in batches of 16 loads, every load of a batch in
        // flight together
        constexpr int DTB = 16 / EK;
#pragma unroll 1
        for (int d0 = 0; d0 < DB; d0 += DTB) {
            bf16x8 wf[DTB][EK];
#pragma unroll
            for (int u = 0; u < DTB; ++u) {
                const bf16* wk = a.wk + (int64_t)(cs * DW + 16 * (d0 + u) + l16) * D + hh * DH + 8 * g;
#pragma unroll
                for (int ek = 0; ek < EK; ++ek) wf[u][ek] = *(const bf16x8*)(wk + 32 * ek);
            }
#pragma unroll
            for (int u = 0; u < DTB; ++u) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ek = 0; ek < EK; ++ek) acc = mfma(wf[u][ek], qb[ek], acc);
                const int dt = d0 + u, row = hs * 16 + l16, ck = (2 * dt + (g >> 1)) ^ l16;
                lds_st_b4(my_ring + (uint32_t)(row * ROWB + ck * 16 + (g & 1) * 8), to_bf16x4(acc));
            }
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int row = hs * 16 + l16, ck = (4 * kc + g) ^ l16;
            uf[kc] = lds_ld8(my_ring + (uint32_t)(row * ROWB + ck * 16));
        }
        // the ring is about to be refilled: both waves of the slice are done
        // with it
        wait_lgkm0();
        block_barrier();
    }

    // ---- streaming: the two waves of a slice each load half of a stage
    const int64_t xrow = a.x_stride * 2;
    const unsigned char* Xg = (const unsigned char*)a.X + ((int64_t)row0 * a.x_stride + (int64_t)cs * DW) * 2;
    auto issue = [&](int t) {
        const uint32_t dst = my_ring + (uint32_t)((t & 1) * STAGE);
        const unsigned char* src = Xg + (int64_t)t * 32 * xrow;
        const int last = nrows - 1 - t * 32;   // rows past the block's end re-read its last row
#pragma unroll
        for (int i = 0; i < OPW; ++i) {
            const int d = 2 * i + hs;
            const int row = 2 * d + (lane >> 5);          // one op = two 512-byte rows
            const int ck = (lane & 31) ^ stca_swz(row);
            const int rr = min(row, last);
            dma16c(src, (uint32_t)(rr * (uint32_t)xrow + ck * 16), __builtin_amdgcn_readfirstlane(dst + d * 1024));
        }
    };

    // per-lane LDS offsets inside a stage.  Score operand: row l16, chunk
    // 4 kc + g; with sw = swz(l16) its swizzled position is
    // 4 (kc ^ (sw >> 2)) + (g ^ (sw & 3)), i.e. base[kc & 3] + 256 (kc >> 2).
    const int sw = stca_swz(l16);
    uint32_t xa[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) xa[m] = (uint32_t)(l16 * ROWB + 64 * (m ^ (sw >> 2)) + 16 * (g ^ (sw & 3)));
    // transposed reads: row 4 g + kq, channels 16 db + 4 q (+0..3); the row's
    // swizzle is 2 v + (g >> 1) with v = 4 (g & 1) + kq, so chunk pair db sits
    // at pair db ^ v: tb8[db & 7] + 256 (db >> 3)
    uint32_t tb8[8];
    {
        const int kq = l16 >> 2, q = l16 & 3, row = 4 * g + kq, v = 4 * (g & 1) + kq;
#pragma unroll
        for (int m = 0; m < 8; ++m)
            tb8[m] = (uint32_t)(row * ROWB + 32 * (m ^ v) + 16 * ((q >> 1) ^ (g >> 1)) + 8 * (q & 1));
    }
    // exchange slot of (slice k, row half r, head hs): [k][2 r + hs]; the
    // partials of the other three slices, in slice order
    uint32_t xo[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) xo[k] = (uint32_t)((k + (k >= cs ? 1 : 0)) * 4 * 64 * 16 + lane * 16);

    // Softmax state per lane (target l16), in log2 units.  The fast loop
    // keeps the maximum at M = 0: weights 2^(s c) are used as long as a
    // lane's tile sum stays within [2^-32, 2^32] (scores of usual scale are far
    // inside), so the accumulator is only ever written by MFMAs.  A wave whose
    // tile falls outside that range (or holds NaN or Inf) finishes the block in
    // the exact loop: running maximum, rescaled accumulator.  Both loops meet
    // the block barrier once per tile at the same point, so waves may switch
    // independently.
    float Mc = 0.f, Zs = 0.f;
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const float c = a.c;

    // Software pipeline, per wave: the scores of tile t+1 are computed while
    // the weights of tile t are formed, and tile t+1's transposed operands
    // are read after tile t's aggregation.
    //   stage_scores(k): partial scores S(k) over the slice -> s (tile k was
    //                    certified by the barrier of stage_tail(k - 1))
    //   stage_tail(k):   X^T(k) -> lo/hi, S(k) -> exchange buffer k & 1; this
    //                    wave's part of tile k + 1 landed; block barrier (both
    //                    waves of a slice are done with slot k & 1, and tile
    //                    k + 1 is complete); slot k & 1 refilled with tile k + 2
    //   iteration t:     full scores of t from the exchange, stage_scores(t+1),
    //                    weights of t, aggregation of t, stage_tail(t+1)
    // The last iteration runs both stages on stale ring data (results unused),
    // so every wave meets ntiles + 1 barriers whichever loop it is in.
    i16x4 lo[DB], hi[DB];
    f32x4 s[2], tot[2];
    auto stage_scores = [&](int k) {
        const uint32_t st = my_ring + (uint32_t)((k & 1) * STAGE);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const uint32_t ad = st + xa[kc & 3] + 256 * (kc >> 2);
            const bf16x8 x0 = lds_ld8(ad);
            const bf16x8 x1 = lds_ld8(ad + 16 * ROWB);
            const f32x4 z0 = kc == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : s[0];
            const f32x4 z1 = kc == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : s[1];
            s[0] = mfma(x0, uf[kc], z0);
            s[1] = mfma(x1, uf[kc], z1);
        }
    };
    auto stage_tail = [&](int k) {
        const uint32_t st = my_ring + (uint32_t)((k & 1) * STAGE);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint32_t ad = st + tb8[db & 7] + 256 * (db >> 3);
            lo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)ad);
            hi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(ad + 16 * ROWB));
        }
        const uint32_t xb = xch_lds + (uint32_t)((k & 1) * NW * 4 * 64 * 16);
#pragma unroll
        for (int r = 0; r < 2; ++r)
            lds_st4(xb + (uint32_t)((cs * 4 + 2 * r + hs) * 64 * 16 + lane * 16), s[r]);
        // every read of slot k & 1 is done, the partials are in place, and
        // this wave's part of tile k + 1 (the only load in flight) has landed
        wait_lgkm0();
        wait_vm<0>();
        block_barrier();
        if (k + 2 < ntiles) issue(k + 2);
    };
    auto read_exchange = [&](int t) {
        const uint32_t xb = xch_lds + (uint32_t)((t & 1) * NW * 4 * 64 * 16);
        f32x4 l[3][2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int k = 0; k < 3; ++k) l[k][r] = lds_ld4(xb + xo[k] + (2 * r + hs) * 64 * 16);
#pragma unroll
        for (int r = 0; r < 2; ++r) tot[r] = ((tot[r] + l[0][r]) + l[1][r]) + l[2][r];
    };
    // (alpha X)^T over the slice's channels += X^T p^T
    auto aggregate = [&](const bf16x8& pk) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            union {
                i16x4 h[2];
                bf16x8 v;
            } vt;
            vt.h[0] = lo[db];
            vt.h[1] = hi[db];
            acc[db] = mfma(vt.v, pk, acc[db]);
        }
    };
    // rows of tile t inside the lane's window: bit j <-> row tok_of(g, j)
    auto valid_bits = [&](int t) {
        uint32_t vj = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = t * 32 + tok_of(g, j);
            vj |= (r >= qlo && r < qhi) ? (1u << j) : 0u;
        }
        return vj;
    };

    if (ntiles > 0) {
        issue(0);
        if (ntiles > 1) issue(1);
        // tile 0 complete for both waves of the slice (tile 1 may be in flight)
        if (ntiles > 1) wait_vm<OPW>();
        else wait_vm<0>();
        block_barrier();
        stage_scores(0);
        stage_tail(0);
    }
    int t = 0;
    for (; t < ntiles; ++t) {
        // the wave's own partial of tile t is still in s: start the sum with it
        tot[0] = s[0];
        tot[1] = s[1];
        read_exchange(t);
        // unconditional (the last tile's extra stage reads stale ring data
        // and is never used) so the MFMAs interleave with the weights below
        stage_scores(t + 1);
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(tot[j >> 2][j & 3] * c);
        const bool full = t * 32 >= qlo && t * 32 + 32 <= qhi;
        uint32_t vj = 0xffu;
        if (!__all(full)) {
            vj = valid_bits(t);
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = ((vj >> j) & 1) ? p[j] : 0.f;
        }
        const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
        const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
        const bf16x8 pk = cat8(q0, q1, q2, q3);
        const float zt = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
        // false for NaN and Inf too
        const bool fits = zt <= kStcaHiBound && (zt >= kStcaLoBound || vj == 0u);
        if (__builtin_expect(!__all(fits), 0)) break;
        Zs += zt;
        aggregate(pk);
        stage_tail(t + 1);
    }
    // exact loop, entered after the scores of tile t + 1 (if any) are in s
    for (bool resume = true; t < ntiles; ++t, resume = false) {
        if (!resume) {
            tot[0] = s[0];
            tot[1] = s[1];
            read_exchange(t);
            stage_scores(t + 1);
        }
        const uint32_t vj = valid_bits(t);
        float x[8];
        float tm = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[j] = ((vj >> j) & 1) ? tot[j >> 2][j & 3] * c : -INFINITY;
            tm = fmaxf(tm, x[j]);
        }
        tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
        // with no weight accumulated yet the maximum may also move down
        const float Mold = Mc;
        const float Mnew = Zs > 0.f ? fmaxf(Mold, tm) : tm;
        const float f = (Zs > 0.f && Mnew != Mold) ? __builtin_amdgcn_exp2f(Mold - Mnew) : 1.f;
        float pe[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pe[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(x[j] - Mnew) : 0.f;
        const bf16x2 q0 = pack2(pe[0], pe[1]), q1 = pack2(pe[2], pe[3]);
        const bf16x2 q2 = pack2(pe[4], pe[5]), q3 = pack2(pe[6], pe[7]);
        const bf16x8 pk = cat8(q0, q1, q2, q3);
        Zs = fmaf(Zs, f, dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f)))));
        if (tm != -INFINITY || Zs > 0.f) Mc = Mnew;
        if (f != 1.f) {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= f;
        }
        aggregate(pk);
        stage_tail(t + 1);
    }
    wait_lgkm0();
    // both waves of the slice are done with its ring before it stages the output
    block_barrier();

    // ---- epilogue: y = acc / Z in bf16, staged through the slice's ring as
    // [head hs * 16 + target][channel] (rows swizzled by target; the two
    // heads' waves write disjoint rows) and written row by row: 512
    // contiguous bytes per row
    {
        float z = Zs;
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        const float inv = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int row = hs * 16 + l16, ck = (2 * db + (g >> 1)) ^ l16;
            lds_st_b4(my_ring + (uint32_t)(row * ROWB + ck * 16 + (g & 1) * 8), to_bf16x4(acc[db] * inv));
        }
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int tt = 2 * it + (lane >> 5), row = hs * 16 + tt, c2 = lane & 31;
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(
            my_ring + (uint32_t)(row * ROWB + ((c2 ^ tt) * 16)));
        if (tt < nt) *(u32x4*)(a.y + ((int64_t)(tb + tt) * a.h + hh) * D + cs * DW + 8 * c2) = v;
    }
}

// One block: the block table (user b gets ceil(targets_b / 16) x (h / 2)
// consecutive entries, in user order) and zero y rows for targets outside
// every user.
__global__ __launch_bounds__(1024) void sa_stca_prep_kernel(StcaArgs a) {
    __shared__ int scan[1024];
    const int tid = threadIdx.x;
    const int hpn = a.h / 2;
    int running = 0;
    for (int base = 0; base < a.B; base += 1024) {
        const int b = base + tid;
        int n = 0;
        if (b < a.B) {
            const int nT = a.tcu[b + 1] - a.tcu[b];
            n = nT > 0 ? (nT + kStcaTargets - 1) / kStcaTargets * hpn : 0;
        }
        scan[tid] = n;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {
            const int v = tid >= o ? scan[tid - o] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        const int start = running + scan[tid] - n;
        if (n > 0) {
            const int u0 = a.cu[b], nu = a.cu[b + 1] - u0, t0 = a.tcu[b], nT = a.tcu[b + 1] - t0;
            for (int c = 0; c * hpn < n; ++c) {
                // the union of the chunk's target windows (clipped to the user)
                const int tb = t0 + c * kStcaTargets, nt = min(kStcaTargets, nT - c * kStcaTargets);
                int lo = nu, hi = 0;
                for (int k = 0; k < nt; ++k) {
                    int wlo = 0, whi = nu;
                    if (a.win != nullptr) {
                        wlo = min(max(a.win[2 * (int64_t)(tb + k)], 0), nu);
                        whi = max(wlo, min(max(a.win[2 * (int64_t)(tb + k) + 1], 0), nu));
                    }
                    if (whi > wlo) {
                        lo = min(lo, wlo);
                        hi = max(hi, whi);
                    }
                }
                const int rows = max(0, hi - lo);
                for (int p = 0; p < hpn; ++p) {
                    const int L = start + c * hpn + p;
                    if (L < a.grid) {
                        a.table[2 * L] = make_int4(b, tb, nt, p);
                        a.table[2 * L + 1] = make_int4(u0 + (rows > 0 ? lo : 0), rows, 0, 0);
                    }
                }
            }
        }
        running += scan[1023];
        __syncthreads();
    }
    for (int L = running + tid; L < a.grid; L += 1024) a.table[2 * L] = make_int4(-1, 0, 0, 0);
    const int t_lo = a.B > 0 ? min(max(a.tcu[0], 0), a.T) : a.T;
    const int t_hi = a.B > 0 ? min(max(a.tcu[a.B], t_lo), a.T) : a.T;
    const int64_t per = (int64_t)a.h * a.D / 8;    // 16-byte chunks of one target's y rows
    for (int64_t i = tid; i < (int64_t)t_lo * per; i += 1024) ((u32x4*)a.y)[i] = (u32x4){0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)t_hi * per + tid; i < (int64_t)a.T * per; i += 1024)
        ((u32x4*)a.y)[i] = (u32x4){0u, 0u, 0u, 0u};
}

bool stca_supported(int D, int dh) { return D == 1024 && (dh == 64 || dh == 128); }

hipError_t launch_stca(const StcaArgs& a, int dh, hipStream_t s) {
    hipLaunchKernelGGL(sa_stca_prep_kernel, dim3(1), dim3(1024), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dh == 64) hipLaunchKernelGGL((sa_stca_kernel<1024, 64>), dim3(a.grid), dim3(2 * kStcaWaves * 64), 0, s, a);
    if (dh == 128) hipLaunchKernelGGL((sa_stca_kernel<1024, 128>), dim3(a.grid), dim3(2 * kStcaWaves * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
