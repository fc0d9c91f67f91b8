// sa_stream_d128.hip -- the streaming Sketch Attention forward on the history
// axis for heads of width 128 (the production shape of appendix G of the
// SequenceO1 paper: one head, d = 128, k = 1024 prototypes), on gfx950.
//
// The computation is the FlashSA one of section 4.4 (score blocks, running
// softmax statistics and aggregation fused; the score matrix never leaves
// registers), arranged as the dh <= 64 streaming kernel arranges it -- row
// ranges split into per-user segments, K and V streamed through an LDS ring by
// direct-to-LDS loads, one wave per 32 prototypes, S^T = K P^T and
// O^T += V^T p^T on v_mfma_f32_16x16x32_bf16 -- with one change that matters
// at this width.  A 32-row stage costs a wave 32 MFMAs (512 cycles of the
// SIMD's matrix unit) and about 65 other vector instructions (the 16 exps
// among them), and on this chip a wave's MFMAs overlap its own independent
// vector instructions but hardly another wave's.  In a plain stage every
// vector instruction depends on the stage's score products and feeds its
// aggregation products, so nothing overlaps.  Here each step of the stage
// loop forms the weights of stage t while the score products of stage t + 1
// run (they depend only on the prototypes and K), then aggregates stage t:
//   step t: weights(t) || scores(t + 1) (K fragments read in step t - 1),
//           V^T(t) reads; [barrier: stage t + 2 in LDS, slot t free] issue
//           stage t + kS into slot t, read K(t + 2); aggregate(t).
// The scores of stage t + 1 are taken against the running maximum as it was
// before stage t's weights; on the rare exact path, where stage t moves the
// maximum from M to M', they are shifted by M - M' (fp32 adds) so that the
// next step sees them relative to M'.
//
// Block = one row range x 256 prototypes of one head (8 waves, two per SIMD,
// one block per CU: a wave needs up to 256 registers), m / 256 blocks per
// head.  The ring holds kS stages of K and V (16 KB each); a step reads two
// of them, and up to kS - 2 are in flight.  Four slots measured fastest
// (three to eight tried: deeper rings were 1-3 % slower).
#include "sa_device.h"
#include "sa_stream_d128.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kS = 4;                      // ring slots
constexpr int kNW = 8;                     // waves per block
constexpr int kDH = 128;
constexpr int kCPR = kDH / 8;              // 16-byte chunks per row per tensor
constexpr int kROWB = kCPR * 16;           // bytes per row per tensor
constexpr int kSTAGE = 32 * kROWB;         // bytes per tensor per stage (8 KB)
static_assert(32 * kCPR == kNW * 64, "one 1 KB DMA op per wave per tensor per stage");

template <bool B>
struct Tag {
    static constexpr bool value = B;
};
using Next = Tag<true>;    // a step followed by the next stage's scores
using Last = Tag<false>;   // the segment's last stage

}  // namespace

template <bool MASKED, bool EXACT>
__global__ __launch_bounds__(kNW * 64, 2) void sa_bf16_stream_d128_kernel(FwdArgs a) {
    constexpr int S = kS;
    constexpr int ROWB = kROWB, STAGE = kSTAGE;
    constexpr int VMS = 2 + (MASKED ? 1 : 0);   // vector-memory ops per wave per stage
    constexpr int FK = 16;                      // K swizzle period (rows)
    constexpr int FV = 8;                       // V swizzle period (rows), chunk pairs
    constexpr int NSB = 2, KC = kDH / 32, DB = kDH / 16;
    static_assert((S - 2) * VMS < 64, "ring depth");

    __shared__ __attribute__((aligned(1024))) unsigned char ring[S][2][STAGE];
    // with a mask: each wave's own copy of a stage's mask bytes, lane i < 32
    // holding the 4-byte word that contains row i's byte
    __shared__ __attribute__((aligned(16))) uint32_t mkring[MASKED ? S : 1][MASKED ? kNW * 64 : 1];

    if (offsets_rejected(a.status)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;

    // (row range w, prototype group gy) of this block, XCD-aware as in the
    // dh <= 64 kernel: with G a multiple of 8 every group of range w runs on
    // XCD w % 8, so the m / 256 blocks that read the same rows share an L2
    int w, gy;
    if (gridDim.x % 8 == 0) {
        const int L = blockIdx.y * gridDim.x + blockIdx.x;
        const int q = L / (8 * gridDim.y), r = L % (8 * gridDim.y);
        w = 8 * q + r % 8;
        gy = r / 8;
    } else {
        w = blockIdx.x;
        gy = blockIdx.y;
    }
    const int bph = a.m / (32 * kNW);           // blocks per head
    const int head = gy / bph;
    const int pb = (gy % bph) * kNW + wave;     // this wave's 32-prototype block

    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, a.split);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);

    const bf16* Pg = (const bf16*)a.P;
    const unsigned char* Kg = (const unsigned char*)a.K;
    const unsigned char* Vg = (const unsigned char*)a.V;
    const int64_t krow = a.k_stride * 2, vrow = a.v_stride * 2;   // bytes between rows

    // prototype fragments, scale * log2(e) folded in (rounded to bf16 once),
    // so that the score products are base-2 scores; with EXACT unscaled: the
    // products are raw scores s (as is the running maximum M below), weights
    // 2^(c (s - M)) and the stored maximum c M
    bf16x8 pf[NSB][KC];
    auto load_p = [&](int b) {
        const bf16* base = Pg + (int64_t)b * a.q_batch_stride + ((int64_t)head * a.m + pb * 32) * kDH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 v = *(const bf16x8*)(base + (int64_t)(16 * sb + l16) * kDH + 32 * kc + 8 * g);
                if constexpr (EXACT) {
                    pf[sb][kc] = v;
                    continue;
                }
                bf16x8 q;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2 t = pack2((float)v[e] * a.c, (float)v[e + 1] * a.c);
                    q[e] = t[0];
                    q[e + 1] = t[1];
                }
                pf[sb][kc] = q;
            }
        wait_vm<0>();
    };
    if (a.q_batch_stride == 0) load_p(0);

    // DMA geometry: lane writes 16 B at LDS offset wave*1024 + lane*16 of a
    // tensor's stage = row * ROWB + slot * 16, fetching the global chunk that
    // the swizzle places in that slot
    const int dma_row = wave * 4 + (lane >> 4);
    const int dslot = lane & 15;
    const uint32_t koff = (uint32_t)(dma_row * (int)krow + (dslot ^ (dma_row % FK)) * 16);
    const uint32_t voff = (uint32_t)(dma_row * (int)vrow + (dslot ^ (2 * (dma_row % FV))) * 16);
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0][0];
    const uint32_t mk_lds = (uint32_t)(uintptr_t)(lds_void*)&mkring[0][0];
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    lds_bf16x8* klane[KC];   // K operand reads, slot 0
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int row = l16, c = 4 * kc + g;
        klane[kc] = (lds_bf16x8*)(uintptr_t)(ring_lds + row * ROWB + ((c ^ (row % FK)) * 16));
    }
    lds_i16x4* vlane[DB];    // V^T transposed reads, slot 0
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int kq = l16 >> 2, q = l16 & 3;
        const int row = 4 * g + kq, colb = (16 * db + 4 * q) * 2;
        vlane[db] = (lds_i16x4*)(uintptr_t)(ring_lds + STAGE + row * ROWB + (((colb >> 4) ^ (2 * (row % FV))) * 16) +
                                            (colb & 15));
    }

    int b = a.users.find_wave(v_lo);
    for (; b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        if (a.q_batch_stride != 0) load_p(b);
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int64_t nrows = s_hi - s_lo;
        const int ntiles = (int)((nrows + 31) / 32);
        const int nrows32 = (int)nrows;
        const unsigned char* kseg = uniform_ptr(Kg + gbase * krow + (int64_t)head * kDH * 2);
        const unsigned char* vseg = uniform_ptr(Vg + gbase * vrow + (int64_t)head * kDH * 2);

        // ---- issue stage t into ring slot `slot` (= t % S): stages are issued
        // in order, so the wave-uniform bases advance by 32 rows per stage; in
        // the last stage rows past the segment end re-read its last row
        const unsigned char* knext = kseg;
        const unsigned char* vnext = vseg;
        auto issue = [&](int t, int slot) {
            const uint32_t slot_lds = ring_lds + (uint32_t)(slot * 2 * STAGE) + (uint32_t)(wave * 1024);
            const int r0 = t * 32;
            const int last = nrows32 - 1 - r0;
            const unsigned char* kb = knext;
            const unsigned char* vb = vnext;
            knext += 32 * krow;
            vnext += 32 * vrow;
            uint32_t ko = koff, vo = voff;
            if (last < 31) {
                const int over = max(dma_row - last, 0);
                ko -= (uint32_t)(over * (int)krow);
                vo -= (uint32_t)(over * (int)vrow);
            }
            dma16s(kb, ko, __builtin_amdgcn_readfirstlane(slot_lds));
            dma16s(vb, vo, __builtin_amdgcn_readfirstlane(slot_lds + STAGE));
            if constexpr (MASKED) {
                // lane -> row (lane % 32) clamped to the segment; the load takes
                // the aligned 4-byte word holding the row's mask byte
                const uintptr_t m0 = (uintptr_t)(a.mask + gbase + r0);
                const int rr = min(lane & 31, last);
                dma4c((const void*)(m0 & ~(uintptr_t)3), (uint32_t)((int)(m0 & 3) + rr) & ~3u,
                      __builtin_amdgcn_readfirstlane(mk_lds + (uint32_t)((slot * kNW + wave) * 256)));
            }
        };
        // validity bits of stage t (32 rows): rows past the segment end or masked are 0
        auto unit_valid = [&](int t, int slot) -> uint32_t {
            const int64_t r0 = (int64_t)t * 32;
            const int rows_here = (int)min((int64_t)32, nrows - r0);
            bool v = lane < rows_here;
            if constexpr (MASKED) {
                const uint32_t m0 = (uint32_t)((uintptr_t)(a.mask + gbase + r0) & 3);
                const int sh = 8 * (int)((m0 + (uint32_t)min(lane & 31, rows_here - 1)) & 3);
                const uint32_t wd = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                    mk_lds + (uint32_t)((slot * kNW + wave) * 256 + 4 * lane));
                v = v && ((wd >> sh) & 0xffu) != 0;
            }
            return (uint32_t)__ballot(v);
        };

        // running maximum M of each of the lane's prototypes, kept negated in
        // the four entries of the tuple that is the first score product's
        // accumulator input (the products come out as s - M); M = 0 and
        // Zs = -1 until the prototype meets a valid row, which sends every
        // stage to the exact path that sets M from the scores
        float Zs[NSB];
        f32x4 nM[NSB];
        f32x4 acc[NSB][DB];
        f32x4 sc[2][NSB];   // scores of the stage whose weights come next
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            nM[sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
            Zs[sb] = -1.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // S^T = K P^T of the stage in `slot` (two 16-row halves), relative to M
        auto scores = [&](int slot, f32x4 (&s)[2][NSB]) {
            const uint32_t sbase = (uint32_t)(slot * 2 * STAGE);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                lds_bf16x8* p0 = klane[kc] + sbase / 16;
                const bf16x8 k0 = p0[0];
                const bf16x8 k1 = p0[16 * ROWB / 16];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const f32x4 z0 = kc == 0 ? nM[sb] : s[0][sb];
                    const f32x4 z1 = kc == 0 ? nM[sb] : s[1][sb];
                    s[0][sb] = mfma(k0, pf[sb][kc], z0);
                    s[1][sb] = mfma(k1, pf[sb][kc], z1);
                }
            }
        };

        // K fragments of the stage in `slot` (8 reads), for its score products
        typedef bf16x8 KFrag[KC][2];
        auto kreads = [&](int slot, KFrag& kf) {
            const uint32_t base = (uint32_t)(slot * 2 * STAGE);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                lds_bf16x8* p0 = klane[kc] + base / 16;
                kf[kc][0] = p0[0];
                kf[kc][1] = p0[16 * ROWB / 16];
            }
        };
        // K fragments of the stage after the one being weighed (read one step
        // ahead, during the previous aggregation, so their latency is hidden)
        KFrag kf;

        // step t: weights and aggregation of stage t (slot).  With NEXT (a
        // stage t + 1 exists) the score products of stage t + 1 run beside the
        // weights; then, once every wave is past its reads of slot t, the
        // barrier that certifies stage t + 2 lets slot t take stage t + S, and
        // stage t + 2's K fragments are read while stage t is aggregated.
        auto step = [&](int t, int slot, int n2slot, auto next_tag) {
            constexpr bool NEXT = decltype(next_tag)::value;
            const uint32_t valid = unit_valid(t, slot);
            const bool seg_full = MASKED ? (t + 1) * 32 <= nrows32 : valid == 0xffffffffu;
            const uint32_t sbase = (uint32_t)(slot * 2 * STAGE);
            const uint32_t vj = lane_slots(valid, g);
            // V^T operands of stage t, read two 16-column blocks at a time
            i16x4 lo[DB], hi[DB];
            auto vreads = [&](int db0) {
#pragma unroll
                for (int db = db0; db < db0 + 2; ++db) {
                    lo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vlane[db] + sbase / 8);
                    hi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vlane[db] + (sbase + 16 * ROWB) / 8);
                }
            };
            // fast-path weights 2^(s - M) of stage t, for the lane's prototypes of
            // block sb and rows h*16 + 4g .. +3 of the stage: 4 exps, 2 packs
            bf16x2 q[NSB][4];
            auto weights = [&](int sb, int h) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(EXACT ? sc[h][sb][i] * a.c : sc[h][sb][i]);
                    if constexpr (MASKED) p[i] = ((vj >> (4 * h + i)) & 1) ? p[i] : 0.f;
                }
                q[sb][2 * h] = pack2(p[0], p[1]);
                q[sb][2 * h + 1] = pack2(p[2], p[3]);
            };
            f32x4 sn[2][NSB];
            if constexpr (NEXT) {
                // four rounds of (one quarter of stage t's weights, stage t + 1's
                // score products of one 32-wide slice of dh, two V^T column
                // blocks), in this order: a wave's vector instructions overlap
                // its own independent MFMAs
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    __builtin_amdgcn_sched_barrier(0);
                    weights(kc >> 1, kc & 1);
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) {
                        const f32x4 z0 = kc == 0 ? nM[sb] : sn[0][sb];
                        const f32x4 z1 = kc == 0 ? nM[sb] : sn[1][sb];
                        sn[0][sb] = mfma(kf[kc][0], pf[sb][kc], z0);
                        sn[1][sb] = mfma(kf[kc][1], pf[sb][kc], z1);
                    }
                    vreads(2 * kc);
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    weights(c >> 1, c & 1);
                    vreads(2 * c);
                }
            }
            // fast path: the running maximum stays, Z += the stage's sum
            bf16x8 pk[NSB];
            // the stage's sums added straight onto Z (the stage's own sum is
            // zn - Z)
            float zn[NSB];
            // lanes whose stage sums fit (false for NaN and Inf too) and whose
            // prototypes have met a valid row, as compare masks (ordered <=
            // and >=) ANDed on the scalar unit: no lane boolean is formed
            uint64_t fits = ~0ull;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                pk[sb] = cat8(q[sb][0], q[sb][1], q[sb][2], q[sb][3]);
                zn[sb] = dot2sum(q[sb][3], dot2sum(q[sb][2], dot2sum(q[sb][1], dot2sum(q[sb][0], Zs[sb]))));
                fits &= __builtin_amdgcn_fcmpf(zn[sb] - Zs[sb], kLazyBound, 5) & __builtin_amdgcn_fcmpf(Zs[sb], 0.f, 3);
            }
            // rare exact path: validity, running-maximum update, rescale
            if (__builtin_expect(!(fits == ~0ull && seg_full), 0)) {
                // the stage's scores again (its K is still in the ring): the
                // same products as before, so that the fast path need not keep
                // them alive past its exps
                f32x4 sr[2][NSB];
                scores(slot, sr);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const float Mold = -nM[sb][0];
                    const bool none = Zs[sb] < 0.f;         // no valid row met yet
                    float x[8];
                    float tm = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        x[j] = ((vj >> j) & 1) ? sr[j >> 2][sb][j & 3] + Mold : -INFINITY;
                        tm = fmaxf(tm, x[j]);
                    }
                    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
                    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
                    const float Mnew = none ? tm : fmaxf(Mold, tm);
                    const bool found = Mnew != -INFINITY;   // the prototype has a valid row
                    const float Mset = found ? Mnew : 0.f;
                    const float f = none ? 0.f
                                         : (Mset == Mold ? 1.f : __builtin_amdgcn_exp2f(EXACT ? (Mold - Mset) * a.c : Mold - Mset));
                    float p[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(EXACT ? (x[j] - Mset) * a.c : x[j] - Mset) : 0.f;
                    const bf16x2 e0 = pack2(p[0], p[1]), e1 = pack2(p[2], p[3]);
                    const bf16x2 e2 = pack2(p[4], p[5]), e3 = pack2(p[6], p[7]);
                    pk[sb] = cat8(e0, e1, e2, e3);
                    float zt = dot2sum(e3, dot2sum(e2, dot2sum(e1, dot2sum(e0, 0.f))));
                    if (none && !found) zt = -1.f;          // Zs = -1 * 0 - 1 keeps the sentinel
                    zn[sb] = fmaf(Zs[sb], f, zt);
                    nM[sb] = (f32x4){-Mset, -Mset, -Mset, -Mset};
                    if constexpr (NEXT) {
                        // the next stage's products were taken against Mold
                        const float sh = Mold - Mset;
                        sn[0][sb] += sh;
                        sn[1][sb] += sh;
                    }
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[sb][db] *= f;
                }
            }
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) Zs[sb] = zn[sb];
            if constexpr (NEXT) {
                // this wave's reads of slot t (V^T above, K again on the exact
                // path) have completed; wait for its part of stage t + 2 (stages
                // up to t + S - 1 have been issued); the barrier then certifies
                // stage t + 2 and frees slot t for stage t + S
                wait_lgkm0();
                const int after = min(t + S - 1, ntiles - 1) - (t + 2);
                wait_after<S - 3, VMS>(max(0, min(S - 3, after)));
                block_barrier();
                if (t + S < ntiles) issue(t + S, slot);
                if (t + 2 < ntiles) kreads(n2slot, kf);
            }
            if (valid != 0xffffffffu) {
                // rows outside the segment or masked: zero their values (NaN must not leak)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (!((vj >> j) & 1)) lo[db][j] = 0;
                        if (!((vj >> (4 + j)) & 1)) hi[db][j] = 0;
                    }
                }
            }
            // O^T += V^T p^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                union {
                    i16x4 h[2];
                    bf16x8 v;
                } vt;
                vt.h[0] = lo[db];
                vt.h[1] = hi[db];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) acc[sb][db] = mfma(vt.v, pk[sb], acc[sb][db]);
            }
            if constexpr (NEXT) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) sc[h][sb] = sn[h][sb];
            }
        };

        // prologue: all S slots filled (stages 0 .. S - 1), the scores of
        // stage 0 and the K fragments of stage 1
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (i < ntiles) issue(i, i);
        wait_after<S - 1, VMS>(min(S - 1, ntiles - 1));
        block_barrier();
        scores(0, sc);
        if (1 < ntiles) {
            wait_after<S - 2, VMS>(min(S - 2, ntiles - 2));
            block_barrier();
            kreads(1, kf);
        }
        int t = 0;
        // unrolled by the ring size, so that every slot offset is a literal
        for (; t + S < ntiles; t += S) {
#pragma unroll
            for (int i = 0; i < S; ++i) step(t + i, i, (i + 2) % S, Next{});
        }
        // at most S - 1 more steps with a next stage, then the last stage
        for (; t + 1 < ntiles; ++t) {
            const int sl = t % S;
            step(t, sl, sl + 2 >= S ? sl + 2 - S : sl + 2, Next{});
        }
        step(t, t % S, 0, Last{});

        // ---- segment epilogue: partial statistics at slot w + b, the sums in
        // lane order, written through to memory
        {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int j = pb * 32 + 16 * sb + l16;
                const int64_t base = (slot * a.H + head) * a.m + j;
                float z = fmaxf(Zs[sb], 0.f);     // the -1 of a prototype with no valid row
                z += __shfl_xor(z, 16, 64);
                z += __shfl_xor(z, 32, 64);
                if (g == 0) {
                    a.part.M[base] = z > 0.f ? (EXACT ? -nM[sb][0] * a.c : -nM[sb][0]) : -INFINITY;
                    a.part.Z[base] = z;
                }
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    store16_wt((f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, kDH, pb * 2 + sb, db, lane),
                               acc[sb][db]);
            }
        }
        // drain this segment's memory traffic and let every wave finish reading
        // the ring before the next segment's prologue refills it
        wait_vm<0>();
        wait_lgkm0();
        block_barrier();
    }
}

bool stream_d128_config(int m, int H, StreamConfig* cfg) {
    if (m % 256 != 0 || H < 1) return false;
    cfg->PB = m / 32;
    cfg->MB = 32;
    cfg->NH = 1;
    cfg->NW = kNW;
    cfg->groups = H * (m / 256);
    cfg->blocks_per_cu = 1;
    return true;
}

hipError_t launch_stream_d128(const FwdArgs& a, const StreamConfig& cfg, hipStream_t s) {
    if (a.dh != kDH || a.norm != 0 || a.m % 256 != 0 || cfg.groups != a.H * (a.m / 256)) return hipErrorInvalidValue;
    dim3 grid(a.G, cfg.groups), block(kNW * 64);
    if (a.exact_scale) {
        if (a.mask) hipLaunchKernelGGL((sa_bf16_stream_d128_kernel<true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((sa_bf16_stream_d128_kernel<false, true>), grid, block, 0, s, a);
    } else {
        if (a.mask) hipLaunchKernelGGL((sa_bf16_stream_d128_kernel<true, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((sa_bf16_stream_d128_kernel<false, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sa
