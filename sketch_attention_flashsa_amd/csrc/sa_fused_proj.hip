// sa_fused_proj.hip -- fused key/value projection + Sketch Attention forward
// for bf16 history rows X (history axis).
//
// The paper's SA scores prototypes against keys K = X W_K (section 3.1; the
// projection is the 2 L d^2 term of the FLOP count in appendix G.3) and
// aggregates values; here V = X W_V, or V = X itself when no W_V is given
// (section 3.1 "Sketch construction" aggregates X).  K and V are produced
// tile by tile in registers and consumed at once by the streaming softmax of
// section 4.4, so they never reach device memory: the only HBM stream is X.
//
// Block = one row range w (the virtual-row segments of sa_internal.h) x four
// heads, two waves per head, one block (8 waves, 2 per SIMD) per CU.  The two
// waves of a head split the work evenly: wave 0 holds W_K,h and projects K,
// wave 1 holds W_V,h and projects V; each owns half of the m prototypes
// (fragments and m/2 x dh accumulators in registers for the whole launch).
// Per 32-row tile:
//   1. the block's DMA ring brings the tile of X into LDS (global_load_lds,
//      16-byte chunks, XOR-swizzled so the fragment reads are conflict free);
//   2. wave 0: K^T = W_K,h^T X^T, wave 1: V = X W_V,h, on
//      v_mfma_f32_16x16x32_bf16, rounded to bf16 and published in a small
//      double-buffered LDS exchange;
//   3. the results are already in the operand layouts of the next two
//      products, up to one fixed permutation of the 32-long contraction index
//      (k-slot j of lane group g holds index tok_of(g, j)); the prototype
//      fragments are loaded in that permuted order, so no data moves between
//      lanes.  One step later (after the next barrier) each wave takes its
//      partner's half and runs, for its prototypes: S^T = K P^T, the online
//      softmax (base 2, lazy maximum) per 16-prototype block, O^T += V^T p^T.
//      As in the streaming kernel, the prototypes are pre-scaled by
//      scale * log2(e) (rounded to bf16 once) and the negated running maximum
//      is the score product's accumulator input, so a weight is one exp2.
// The projection of tile t and the softmax of tile t-1 share a step, so one
// barrier per tile orders both the ring and the exchange.  Inside a step the
// projection's products are spread over the prototype blocks: each block
// issues the score products of the next block, its share of the projection
// and the aggregation of the previous block, then forms its own weights, so
// the weights' vector instructions overlap the wave's own matrix products
// (another wave's vector work hardly overlaps them on this chip).  The
// segment loop is compiled once per role, so the two roles' loop-carried
// state never meets at a branch join (which would copy it every tile).
// X is read without the non-temporal hint: the two head groups of a row
// range run on one XCD (blocks w and G + w) and read the same rows, so the
// second read can hit that XCD's L2.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_fold.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kFStages = 4;   // X ring slots: 3 tiles in flight, 1 computed
constexpr int kFWaves = 8;    // waves per block: two per head
// bounds of the running maximum's moves (base-2 exponents): a weight stays
// below 2^kLazyLog2, so a lane's eight weights of a tile stay within
// kLazyBound; the first summed mass of a prototype is at least 2^-kFloorLog2
constexpr float kLazyLog2 = 13.0f;
constexpr float kFloorLog2 = 60.0f;
constexpr float kSumFloor = 8.673617379884035e-19f;   // 2^-60

template <int V>
using Int = std::integral_constant<int, V>;

}  // namespace

template <int DM, int MB, bool MASKED, bool VX>
__global__ __launch_bounds__(kFWaves * 64, 1) void sa_fused_proj_kernel(FusedArgs a) {
    constexpr int DH = 32;
    constexpr int S = kFStages;
    constexpr int ROWB = DM * 2;               // bytes per X row
    constexpr int STAGE = 32 * ROWB;           // one 32-row tile
    constexpr int OPS = STAGE / 1024;          // 1 KB DMA ops per tile
    constexpr int D = OPS / kFWaves;           // per wave
    // with a mask, its words travel with the tile (MDMA) where the LDS has room
    // for them: every shape but d_model = 256 with m = 256, whose ring,
    // exchange and prototypes fill the LDS
    constexpr bool MDMA = MASKED && !(DM == 256 && MB == 128);
    constexpr int VMS = D + (MDMA ? 1 : 0);   // vector-memory ops per wave per tile
    constexpr int AHEAD = S - 1;
    constexpr int KCX = DM / 32;               // 32-wide chunks of the model dimension
    constexpr int NSB = MB / 16;               // prototype blocks of one wave
    constexpr int HPB = kFWaves / 2;           // heads per block
    static_assert(DM == 128 || DM == 256, "model width");
    static_assert(D >= 1 && D * kFWaves == OPS, "whole DMA ops per wave");
    static_assert((AHEAD - 1) * VMS < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) unsigned char ring[S][STAGE];
    // with a mask: each wave's own copy of a tile's mask words, lane i < 32
    // holding the aligned 4-byte word that contains row i's byte (a plain
    // load at the point of use would make the compiler, which cannot count
    // the ring's asm loads, drain the ring)
    __shared__ __attribute__((aligned(16))) uint32_t mkring[MDMA ? S : 1][MDMA ? kFWaves * 64 : 1];
    // exchange: [tile parity][head][role][fragment][lane]
    __shared__ __attribute__((aligned(16))) bf16x8 xchg[2][HPB][2][2][64];

    if (offsets_rejected(a.status)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int hl = wave >> 1, role = wave & 1;       // role 0: K, role 1: V
    const int w = blockIdx.x;
    const int head = blockIdx.y * HPB + hl;
    const bool active = head < a.H;                   // uniform per head pair
    const int hh = active ? head : a.H - 1;           // idle pairs load a valid head's data
    const int pbase = role * MB;                      // first prototype of this wave

    const int64_t total = a.users.total();
    const int64_t R = chunk_rows(total, a.G, a.R_fixed, a.R_min);
    const int64_t v_lo = (int64_t)w * R;
    if (v_lo >= total) return;
    const int64_t v_hi = min(v_lo + R, total);
    const int HD = a.H * DH;

    // ---- this wave's weight fragments: element j of lane (g, l16) in dh
    // block db and chunk kc is W[32 kc + 8 g + j][h dh + 16 db + l16], W = W_K
    // (role 0) or W_V (role 1; the identity's columns when V = X).  Gathered
    // one fragment per iteration through the (not yet used) ring, so few
    // loads are in flight.
    bf16x8 wf[2][KCX];
    {
        static_assert(sizeof(bf16x8) * 64 * KCX * kFWaves <= sizeof(ring), "staging fits the ring");
        bf16x8* stage = (bf16x8*)&ring[0][0] + wave * KCX * 64;
        const bf16* W = (const bf16*)(role == 0 ? a.Wk : a.Wv);
        const bool ident = VX && role == 1;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
#pragma unroll 1
            for (int kc = 0; kc < KCX; ++kc) {
                const int col = hh * DH + 16 * db + l16;
                bf16x8 v;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int k = 32 * kc + 8 * g + j;
                    v[j] = ident ? (bf16)(k == col ? 1.0f : 0.0f) : W[(int64_t)k * HD + col];
                }
                stage[kc * 64 + lane] = v;
            }
#pragma unroll
            for (int kc = 0; kc < KCX; ++kc) wf[db][kc] = stage[kc * 64 + lane];
        }
    }
    // ---- prototype fragments, contraction index permuted: element j of lane
    // (g, l16) in block sb is P[h, pbase + 16 sb + l16, tok_of(g, j)] * c
    // (scale * log2(e), rounded to bf16 once, so the products are base-2
    // scores).  They live in LDS in lane order (one conflict-free 16-byte
    // read each).
    __shared__ __attribute__((aligned(16))) bf16x8 pl[kFWaves][NSB][64];
    auto load_p = [&](int b) {
        const bf16* base = (const bf16*)a.P + (int64_t)b * a.q_batch_stride + ((int64_t)hh * a.m + pbase) * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const bf16* row = base + (int64_t)(16 * sb + l16) * DH;
            const bf16x4 lo = *(const bf16x4*)(row + 4 * g);
            const bf16x4 hi = *(const bf16x4*)(row + 16 + 4 * g);
            const bf16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            bf16x8 q;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 t = pack2((float)v[e] * a.c, (float)v[e + 1] * a.c);
                q[e] = t[0];
                q[e + 1] = t[1];
            }
            pl[wave][sb][lane] = q;
        }
        wait_vm<0>();   // settle before any ring traffic is counted
    };
    if (a.q_batch_stride == 0) load_p(0);
    wait_vm<0>();
    __syncthreads();   // the ring's staging use is over

    // per-lane DMA geometry: op (wave*D + d) writes LDS [op*1024, +1024); lane
    // writes 16 B at row*ROWB + slot*16, fetching chunk slot ^ (row & 15)
    int dma_row[D], dma_off[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int off = (wave * D + d) * 1024 + lane * 16;
        dma_row[d] = off / ROWB;
        const int slot = (off % ROWB) / 16;
        dma_off[d] = (slot ^ (dma_row[d] & 15)) * 16;   // byte offset of the fetched chunk in its row
    }
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0];
    const uint32_t mk_lds = (uint32_t)(uintptr_t)(lds_void*)&mkring[0][0];
    // this lane's X fragment of row block rb and chunk kc sits at row
    // 16 rb + l16, 16-byte position (4 kc + g) ^ l16 = (g ^ (l16 & 3)) +
    // 4 ((kc & 3) ^ (l16 >> 2)) + 16 (kc >> 2) of a ring slot: four lane
    // offsets, one per kc & 3, and immediates for rb and kc >> 2
    uint32_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xoff[i] = (uint32_t)(l16 * ROWB + 16 * (g ^ (l16 & 3)) + 64 * (i ^ (l16 >> 2)));

    const unsigned char* Xg = (const unsigned char*)a.X;

    // the segment loop, compiled once per role so that the two roles' loop
    // state (accumulators, running maxima) never meets at a branch join
    auto segments = [&](auto role_c) {
        constexpr int ROLE = decltype(role_c)::value;
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
            const unsigned char* xseg = Xg + gbase * ROWB;

            // tile t: lane fetches row min(dma_row, last row of the segment) of
            // the tile (rows past the end re-read the last row; they are invalid)
            auto issue = [&](int t) {
                const uint32_t slot_lds = ring_lds + (uint32_t)((t % S) * STAGE) + (uint32_t)(wave * D * 1024);
                const int r0 = t * 32;
                const unsigned char* tbase = xseg + (int64_t)r0 * ROWB;
                const int last = nrows32 - 1 - r0;
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const uint32_t voff = (uint32_t)(min(dma_row[d], last) * ROWB + dma_off[d]);
                    dma16c(tbase, voff, __builtin_amdgcn_readfirstlane(slot_lds + d * 1024));
                }
                if constexpr (MDMA) {
                    // lane -> row (lane % 32) clamped to the segment: the aligned
                    // word around its mask byte (never leaves the byte's page)
                    const uintptr_t m0 = (uintptr_t)(a.mask + gbase + r0);
                    const int rr = min(lane & 31, last);
                    dma4c((const void*)(m0 & ~(uintptr_t)3), (uint32_t)((int)(m0 & 3) + rr) & ~3u,
                          __builtin_amdgcn_readfirstlane(mk_lds + (uint32_t)(((t % S) * kFWaves + wave) * 256)));
                }
            };
            auto tile_valid = [&](int t) -> uint32_t {
                const int64_t r0 = (int64_t)t * 32;
                const int rows_here = (int)min((int64_t)32, nrows - r0);
                bool v = lane < rows_here;
                if constexpr (MDMA) {
                    // the tile's mask words arrived with it (this wave's own copy)
                    const uint32_t m0 = (uint32_t)((uintptr_t)(a.mask + gbase + r0) & 3);
                    const int sh = 8 * (int)((m0 + (uint32_t)min(lane & 31, rows_here - 1)) & 3);
                    const uint32_t wd = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                        mk_lds + (uint32_t)(((t % S) * kFWaves + wave) * 256 + 4 * lane));
                    v = v && ((wd >> sh) & 0xffu) != 0;
                } else if constexpr (MASKED) {
                    v = v && a.mask[gbase + r0 + min(lane, rows_here - 1)] != 0;
                }
                return (uint32_t)__ballot(v);
            };

            // the running maximum M of each of the lane's prototypes is kept
            // negated and broadcast into the score products' accumulator input
            // (one scalar per block: the four-wide tuples would not fit beside
            // the weight fragments).  Every M starts at 0 and moves only when
            // a tile's weights 2^(s - M) would leave the range the sums keep
            // exact (see the exact path), so with scores of usual size it stays
            // 0 for the whole segment; while all of the wave's maxima are 0
            // (mz) the products take the constant 0 as accumulator input and
            // no tuple is built.  Zs = 0 until the prototype meets a valid row.
            float nM[NSB];
            float Zs[NSB];
            f32x4 acc[NSB][2];
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                nM[sb] = 0.f;
                Zs[sb] = 0.f;
                acc[sb][0] = acc[sb][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
            // wave-uniform: every nM of this wave is 0.  With a mask most tiles
            // hold an excluded row and take the exact path anyway, so masked
            // instances run the general loop alone (one loop: no spills)
            bool mz = !MASKED;

            // one step t: the softmax of tile t - 1 (ATT; its K and V were
            // published in step t - 1) and the projection of tile t (PROJ), the
            // projection's products spread over the prototype blocks beside each
            // block's weights: only a wave's own vector instructions overlap its
            // matrix products.  Projection unit u = (chunk kc = u / 2, row block
            // rb = u % 2): one X fragment, two products.
            constexpr int UPB = 2 * KCX / NSB;   // projection units per prototype block
            static_assert(UPB >= 1 && UPB * NSB == 2 * KCX, "projection units per block");
            uint32_t valid_prev = 0;
            bf16x8 pn[2];                         // prototype blocks 0 and 1, read at the end of the step before
            pn[0] = pl[wave][0][lane];
            pn[1] = pl[wave][NSB > 1 ? 1 : 0][lane];
            auto xread = [&](int t, int u) {
                const int kc = u >> 1, rb = u & 1;
                const uint32_t slot = ring_lds + (uint32_t)((t % S) * STAGE);
                return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(
                    slot + xoff[kc & 3] + (uint32_t)(rb * 16 * ROWB + 256 * (kc >> 2)));
            };
            auto step = [&](auto att_c, auto proj_c, auto mz_c, int t) {
                constexpr bool ATT = decltype(att_c)::value != 0;
                constexpr bool PROJ = decltype(proj_c)::value != 0;
                constexpr bool MZ = decltype(mz_c)::value != 0;   // all maxima 0: products from 0
                bf16x8 ka[2], vt[2];
                if constexpr (ATT) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        ka[i] = xchg[(t - 1) & 1][hl][0][i][lane];
                        vt[i] = xchg[(t - 1) & 1][hl][1][i][lane];
                    }
                }
                const uint32_t vj = lane_slots(valid_prev, g);
                const uint32_t valid = PROJ ? tile_valid(t) : 0u;
                // projection accumulators: role 0 K^T[db][rb], role 1 V[rb][db]
                f32x4 r[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i) r[i][0] = r[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
                auto punit = [&](int u, const bf16x8& xf) {
                    const int kc = u >> 1, rb = u & 1;
#pragma unroll
                    for (int db = 0; db < 2; ++db) {
                        if constexpr (ROLE == 0) r[db][rb] = mfma(wf[db][kc], xf, r[db][rb]);
                        else r[rb][db] = mfma(xf, wf[db][kc], r[rb][db]);
                    }
                };
                // the first block's X fragments; the others are read in their
                // block (one block ahead would not fit the registers)
                bf16x8 xq[UPB];
                if constexpr (PROJ) {
#pragma unroll
                    for (int i = 0; i < UPB; ++i) xq[i] = xread(t, i);
                }
                // prototype fragments: block sb's is read during block sb - 2
                bf16x8 pf[NSB];
                pf[0] = pn[0];
                if constexpr (NSB > 1) pf[1] = pn[1];
                // base-2 scores minus the running maximum of block sb
                auto scores = [&](int sb, f32x4& s0, f32x4& s1) {
                    if constexpr (MZ) {
                        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
                        s0 = mfma(ka[0], pf[sb], z4);
                        s1 = mfma(ka[1], pf[sb], z4);
                        return;
                    }
                    float m1 = nM[sb];
                    asm volatile("" : "+v"(m1));   // rebuilt per use, not hoisted
                    const f32x4 c4 = {m1, m1, m1, m1};
                    s0 = mfma(ka[0], pf[sb], c4);
                    s1 = mfma(ka[1], pf[sb], c4);
                };
                f32x4 s0, s1;
                if constexpr (ATT) scores(0, s0, s1);
                bf16x8 pkp;   // the previous block's weights, aggregated one block late
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    // the products of block sb + 1, a share of the projection and
                    // the aggregation of block sb - 1 go before the weights of
                    // block sb, which then overlap them (a block's running maximum
                    // and sums are its own, so the exact path of sb touches none)
                    __builtin_amdgcn_sched_barrier(0);
                    f32x4 s0n, s1n;
                    if constexpr (ATT) {
                        if (sb + 1 < NSB) scores(sb + 1, s0n, s1n);
                        if (sb + 2 < NSB) pf[sb + 2] = pl[wave][sb + 2][lane];
                    }
                    if constexpr (PROJ) {
#pragma unroll
                        for (int i = 0; i < UPB; ++i) punit(sb * UPB + i, sb == 0 ? xq[i] : xread(t, sb * UPB + i));
                    }
                    if constexpr (ATT) {
                        if (sb > 0) {
                            acc[sb - 1][0] = mfma(vt[0], pkp, acc[sb - 1][0]);
                            acc[sb - 1][1] = mfma(vt[1], pkp, acc[sb - 1][1]);
                        }
                        float p[8];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            p[j] = __builtin_amdgcn_exp2f(s0[j]);
                            p[4 + j] = __builtin_amdgcn_exp2f(s1[j]);
                        }
                        const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                        const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                        bf16x8 pk = cat8(q0, q1, q2, q3);
                        // fast path: the running maximum stays; Z += the tile's sum,
                        // summed straight onto Z (the tile's own sum is znew - Z)
                        float znew = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, Zs[sb]))));
                        // lanes whose tile sum fits (false for NaN and Inf too) and
                        // whose running sum is clear of underflow, as compare masks
                        // (ordered <= and >=), so no lane boolean is formed
                        const uint64_t fits = __builtin_amdgcn_fcmpf(znew - Zs[sb], kLazyBound, 5) &
                                              __builtin_amdgcn_fcmpf(znew, kSumFloor, 3);
                        // rare exact path (then-only, so the common path keeps its
                        // values in place): validity, running-maximum update, rescale
                        if (__builtin_expect(!(fits == ~0ull && valid_prev == 0xffffffffu), 0)) {
                            // scores relative to 0 again (the products held s - M)
                            const float Mold = -nM[sb];
                            const bool none = !(Zs[sb] > 0.f);      // no valid row met yet
                            float x[8];
                            float tm = -INFINITY;
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const float sv = j < 4 ? s0[j] : s1[j - 4];
                                x[j] = ((vj >> j) & 1) ? sv + Mold : -INFINITY;
                                tm = fmaxf(tm, x[j]);
                            }
                            tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
                            tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
                            // the maximum moves to the tile's only where it must: when a
                            // weight 2^(s - M) of the tile could exceed 2^kLazyLog2 (eight
                            // of them per lane stay within the fast path's bound), or,
                            // before any mass is summed, when the largest would fall
                            // below 2^-kFloorLog2 (with no valid row tm is -inf: M stays)
                            const bool up = tm > Mold + kLazyLog2;
                            const bool low = none && tm < Mold - kFloorLog2;
                            const float Mset = (tm != -INFINITY && (up || low)) ? tm : Mold;
                            if constexpr (MZ) {
                                if (__ballot(Mset != 0.f) != 0) mz = false;
                            }
                            const float f = none ? 0.f : (Mset == Mold ? 1.f : __builtin_amdgcn_exp2f(Mold - Mset));
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(x[j] - Mset) : 0.f;
                            const bf16x2 e0 = pack2(p[0], p[1]), e1 = pack2(p[2], p[3]);
                            const bf16x2 e2 = pack2(p[4], p[5]), e3 = pack2(p[6], p[7]);
                            pk = cat8(e0, e1, e2, e3);
                            const float zadd = dot2sum(e3, dot2sum(e2, dot2sum(e1, dot2sum(e0, 0.f))));
                            nM[sb] = -Mset;
                            acc[sb][0] *= f;
                            acc[sb][1] *= f;
                            znew = fmaf(Zs[sb], f, zadd);
                        }
                        Zs[sb] = znew;
                        pkp = pk;
                        if (sb + 1 < NSB) {
                            s0 = s0n;
                            s1 = s1n;
                        }
                    }
                }
                if constexpr (ATT) {
                    acc[NSB - 1][0] = mfma(vt[0], pkp, acc[NSB - 1][0]);
                    acc[NSB - 1][1] = mfma(vt[1], pkp, acc[NSB - 1][1]);
                }
                if constexpr (PROJ) {
                    // role 0: q = rb, (K^T[0][rb], K^T[1][rb]); role 1: q = db,
                    // (V[0][db], V[1][db]): slot j <- dh or row tok_of(g, j)
                    bf16x8 own[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        own[q] = cat8(pack2(r[0][q][0], r[0][q][1]), pack2(r[0][q][2], r[0][q][3]),
                                      pack2(r[1][q][0], r[1][q][1]), pack2(r[1][q][2], r[1][q][3]));
                    if constexpr (ROLE == 1) {
                        if (valid != 0xffffffffu) {   // invalid rows' values zeroed
                            const uint32_t vv = lane_slots(valid, g);
#pragma unroll
                            for (int q = 0; q < 2; ++q)
#pragma unroll
                                for (int j = 0; j < 8; ++j)
                                    if (!((vv >> j) & 1)) own[q][j] = (bf16)0.0f;
                        }
                    }
                    xchg[t & 1][hl][ROLE][0][lane] = own[0];
                    xchg[t & 1][hl][ROLE][1][lane] = own[1];
                }
                // the next step's first two prototype blocks
                pn[0] = pl[wave][0][lane];
                if constexpr (NSB > 1) pn[1] = pl[wave][1][lane];
                valid_prev = valid;
            };

#pragma unroll
            for (int t = 0; t < AHEAD; ++t)
                if (t < ntiles) issue(t);

            auto run = [&](auto att_c, auto proj_c, auto mz_c, int t) {
                if (t < ntiles) wait_after<AHEAD - 1, VMS>(min(AHEAD - 1, ntiles - 1 - t));
                block_barrier();
                if (t + AHEAD < ntiles) issue(t + AHEAD);
                if (active) step(att_c, proj_c, mz_c, t);
                // every LDS access of this step has completed before the next barrier
                wait_lgkm0();
            };
            // steps with every maximum at 0, then (once one has moved: a
            // wave-uniform, one-way switch) the general steps
            run(Int<0>{}, Int<1>{}, Int<1>{}, 0);
            int t = 1;
            for (; t < ntiles && mz; ++t) run(Int<1>{}, Int<1>{}, Int<1>{}, t);
            for (; t < ntiles; ++t) run(Int<1>{}, Int<1>{}, Int<0>{}, t);
            if (mz) run(Int<1>{}, Int<0>{}, Int<1>{}, ntiles);
            else run(Int<1>{}, Int<0>{}, Int<0>{}, ntiles);

            // ---- segment epilogue: partial statistics at slot w + b
            if (active) {
                const int64_t slot = (int64_t)w + b;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const int j = pbase + 16 * sb + l16;
                    const int64_t base = (slot * a.H + head) * a.m + j;
                    float z = Zs[sb];                 // 0 for a prototype with no valid row
                    z += __shfl_xor(z, 16, 64);
                    z += __shfl_xor(z, 32, 64);
                    if (g == 0) {
                        // no valid row in the segment: M = -inf, as the merge expects
                        a.part.M[base] = z > 0.f ? -nM[sb] : -INFINITY;
                        a.part.Z[base] = z;
                    }
#pragma unroll
                    for (int db = 0; db < 2; ++db)
                        __builtin_nontemporal_store(acc[sb][db], (f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH,
                                                                                        pbase / 16 + sb, db, lane));
                }
            }
            wait_vm<0>();
            wait_lgkm0();
            block_barrier();
        }
    };
    if (role == 0) segments(Int<0>{});
    else segments(Int<1>{});
}

namespace {

template <int DM, int MB>
void launch_fused_t(const FusedArgs& a, bool masked, bool vx, hipStream_t s) {
    dim3 grid(a.G, fused_groups(a.H)), block(kFWaves * 64);
    if (!masked && !vx) hipLaunchKernelGGL((sa_fused_proj_kernel<DM, MB, false, false>), grid, block, 0, s, a);
    if (masked && !vx) hipLaunchKernelGGL((sa_fused_proj_kernel<DM, MB, true, false>), grid, block, 0, s, a);
    if (!masked && vx) hipLaunchKernelGGL((sa_fused_proj_kernel<DM, MB, false, true>), grid, block, 0, s, a);
    if (masked && vx) hipLaunchKernelGGL((sa_fused_proj_kernel<DM, MB, true, true>), grid, block, 0, s, a);
}

}  // namespace

// P_h W_K,h^T on MFMA (m and d_model multiples of 16, dh of 32): one wave
// per 16 x 16 output tile (prototypes j0.., model channels e0..), the
// operands read straight from memory (both are k-contiguous):
// A = 16 prototype rows of P_h, B = 16 rows of W restricted to head h's
// columns; the lane's four results (prototypes j0 + 4g .. + 3, channel
// e0 + l16) are scaled and rounded once.
__global__ __launch_bounds__(256) void sa_fold_keys_mfma_kernel(const bf16* P, const bf16* W, int H, int m, int dh,
                                                                int d_model, float c, bf16* out) {
    const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int tn = d_model / 16, tm = m / 16;
    if (tile >= (int64_t)H * tm * tn) return;
    const int e0 = (int)(tile % tn) * 16;
    const int64_t hj = tile / tn;
    const int j0 = (int)(hj % tm) * 16, h = (int)(hj / tm);
    const bf16* pa = P + ((int64_t)h * m + j0 + l16) * dh + 8 * g;
    const bf16* wb = W + (int64_t)(e0 + l16) * H * dh + (int64_t)h * dh + 8 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < dh; k += 32)
        acc = mfma(*(const bf16x8*)(pa + k), *(const bf16x8*)(wb + k), acc);
    bf16* o = out + ((int64_t)h * m + j0 + 4 * g) * d_model + e0 + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[(int64_t)r * d_model] = (bf16)(acc[r] * c);
}

hipError_t launch_fold_keys(const bf16* P, const bf16* W, int H, int m, int dh, int d_model, float c, bf16* out,
                            hipStream_t s) {
    const int64_t n = (int64_t)H * m * d_model;
    if (n <= 0) return hipSuccess;
    if (m % 16 != 0 || d_model % 16 != 0 || dh % 32 != 0) return hipErrorInvalidValue;
    const int64_t tiles = (int64_t)H * (m / 16) * (d_model / 16);
    hipLaunchKernelGGL(sa_fold_keys_mfma_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, P, W, H, m, dh,
                       d_model, c, out);
    return hipGetLastError();
}

bool fused_supported(int d_model, int m, int dh) {
    return dh == 32 && (d_model == 128 || d_model == 256) && (m == 64 || m == 128 || m == 256);
}

int fused_groups(int H) { return (H + kFWaves / 2 - 1) / (kFWaves / 2); }

hipError_t launch_fused(const FusedArgs& a, hipStream_t s) {
    const bool masked = a.mask != nullptr, vx = a.Wv == nullptr;
    // each wave of a head pair owns half of the m prototypes
    if (a.d_model == 256) {
        if (a.m == 256) launch_fused_t<256, 128>(a, masked, vx, s);
        else if (a.m == 128) launch_fused_t<256, 64>(a, masked, vx, s);
        else launch_fused_t<256, 32>(a, masked, vx, s);
    } else {
        if (a.m == 256) launch_fused_t<128, 128>(a, masked, vx, s);
        else if (a.m == 128) launch_fused_t<128, 64>(a, masked, vx, s);
        else launch_fused_t<128, 32>(a, masked, vx, s);
    }
    return hipGetLastError();
}

}  // namespace sa
