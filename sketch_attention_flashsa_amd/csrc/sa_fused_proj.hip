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
// The projection of tile t and the softmax of tile t-1 share a step, so one
// barrier per tile orders both the ring and the exchange.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kFStages = 4;   // X ring slots: 3 tiles in flight, 1 computed
constexpr int kFWaves = 8;    // waves per block: two per head

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
    // (g, l16) in block sb is P[h, pbase + 16 sb + l16, tok_of(g, j)].  They
    // live in LDS in lane order (one conflict-free 16-byte read each).
    __shared__ __attribute__((aligned(16))) bf16x8 pl[kFWaves][NSB][64];
    auto load_p = [&](int b) {
        const bf16* base = (const bf16*)a.P + (int64_t)b * a.q_batch_stride + ((int64_t)hh * a.m + pbase) * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const bf16* row = base + (int64_t)(16 * sb + l16) * DH;
            const bf16x4 lo = *(const bf16x4*)(row + 4 * g);
            const bf16x4 hi = *(const bf16x4*)(row + 16 + 4 * g);
            pl[wave][sb][lane] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
    // LDS address of this lane's X fragment (row block 0, chunk 0) in slot 0
    const uint32_t xlane = ring_lds + (uint32_t)(l16 * ROWB);

    const unsigned char* Xg = (const unsigned char*)a.X;

    int b = a.users.find(v_lo);
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
                dma16s(tbase, voff, __builtin_amdgcn_readfirstlane(slot_lds + d * 1024));
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

        float Mc[NSB], Zs[NSB];
        f32x4 acc[NSB][2];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            Mc[sb] = -INFINITY;
            Zs[sb] = 0.f;
            acc[sb][0] = acc[sb][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // projection of tile t by this wave, published in the exchange: role 0
        // the K operands of the two row blocks (slot j <- dh tok_of(g, j)),
        // role 1 the V^T operands of the two dh blocks (slot j <- row
        // tok_of(g, j), invalid rows zeroed)
        auto project = [&](auto role_c, int t, uint32_t valid) {
            constexpr int ROLE = decltype(role_c)::value;
            const uint32_t xb = xlane + (uint32_t)((t % S) * STAGE);
            f32x4 r[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) r[i][0] = r[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KCX; ++kc) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const uint32_t ad = xb + (uint32_t)(rb * 16 * ROWB + (((4 * kc + g) ^ l16) * 16));
                    const bf16x8 xf = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)ad;
#pragma unroll
                    for (int db = 0; db < 2; ++db) {
                        if constexpr (ROLE == 0) r[db][rb] = mfma(wf[db][kc], xf, r[db][rb]);   // K^T[db rows][rb cols]
                        else r[rb][db] = mfma(xf, wf[db][kc], r[rb][db]);                       // V[rb rows][db cols]
                    }
                }
            }
            // role 0: q = rb, (K^T[0][rb], K^T[1][rb]); role 1: q = db, (V[0][db], V[1][db])
            bf16x8 own[2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                own[q] = cat8(pack2(r[0][q][0], r[0][q][1]), pack2(r[0][q][2], r[0][q][3]),
                              pack2(r[1][q][0], r[1][q][1]), pack2(r[1][q][2], r[1][q][3]));
            if constexpr (ROLE == 1) {
                if (valid != 0xffffffffu) {
                    const uint32_t vj = lane_slots(valid, g);
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (!((vj >> j) & 1)) own[q][j] = (bf16)0.0f;
                }
            }
            xchg[t & 1][hl][ROLE][0][lane] = own[0];
            xchg[t & 1][hl][ROLE][1][lane] = own[1];
        };

        // scores, weights and aggregation of one tile for this wave's prototypes
        auto attend = [&](const bf16x8 (&ka)[2], const bf16x8 (&vt)[2], uint32_t valid) {
            const uint32_t vj = lane_slots(valid, g);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const bf16x8 pf = pl[wave][sb][lane];
                const f32x4 s0 = mfma(ka[0], pf, zero);
                const f32x4 s1 = mfma(ka[1], pf, zero);
                float p[8];
                const float nm = -Mc[sb];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p[j] = __builtin_amdgcn_exp2f(fmaf(s0[j], a.c, nm));
                    p[4 + j] = __builtin_amdgcn_exp2f(fmaf(s1[j], a.c, nm));
                }
                const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                bf16x8 pk = cat8(q0, q1, q2, q3);
                // fast path: the running maximum stays; Z += the tile's sum
                float zadd = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
                float f = 1.f;
                const bool fits = zadd <= kLazyBound;   // false for NaN and Inf too
                // rare exact path (then-only, so the common path keeps its
                // values in place): validity, running-maximum update, rescale
                if (__builtin_expect(!(__all(fits) && valid == 0xffffffffu), 0)) {
                    float x[8];
                    float tm = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float sv = j < 4 ? s0[j] : s1[j - 4];
                        x[j] = ((vj >> j) & 1) ? sv * a.c : -INFINITY;
                        tm = fmaxf(tm, x[j]);
                    }
                    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
                    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
                    const float Mold = Mc[sb];
                    const float Mnew = fmaxf(Mold, tm);
                    f = (Mnew == Mold) ? 1.f : __builtin_amdgcn_exp2f(Mold - Mnew);
#pragma unroll
                    for (int j = 0; j < 8; ++j) p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(x[j] - Mnew) : 0.f;
                    const bf16x2 e0 = pack2(p[0], p[1]), e1 = pack2(p[2], p[3]);
                    const bf16x2 e2 = pack2(p[4], p[5]), e3 = pack2(p[6], p[7]);
                    pk = cat8(e0, e1, e2, e3);
                    zadd = dot2sum(e3, dot2sum(e2, dot2sum(e1, dot2sum(e0, 0.f))));
                    Mc[sb] = Mnew;
                    acc[sb][0] *= f;
                    acc[sb][1] *= f;
                }
                Zs[sb] = fmaf(Zs[sb], f, zadd);
                acc[sb][0] = mfma(vt[0], pk, acc[sb][0]);
                acc[sb][1] = mfma(vt[1], pk, acc[sb][1]);
            }
        };

#pragma unroll
        for (int t = 0; t < AHEAD; ++t)
            if (t < ntiles) issue(t);

        uint32_t valid_prev = 0;
        for (int t = 0; t <= ntiles; ++t) {
            if (t < ntiles) wait_after<AHEAD - 1, VMS>(min(AHEAD - 1, ntiles - 1 - t));
            block_barrier();
            if (t + AHEAD < ntiles) issue(t + AHEAD);
            if (active && t > 0) {
                // both halves of tile t-1, published before this barrier
                const bf16x8 ka[2] = {xchg[(t - 1) & 1][hl][0][0][lane], xchg[(t - 1) & 1][hl][0][1][lane]};
                const bf16x8 vt[2] = {xchg[(t - 1) & 1][hl][1][0][lane], xchg[(t - 1) & 1][hl][1][1][lane]};
                attend(ka, vt, valid_prev);
            }
            if (t < ntiles) {
                const uint32_t valid = tile_valid(t);
                if (active) {
                    if (role == 0) project(std::integral_constant<int, 0>{}, t, valid);
                    else project(std::integral_constant<int, 1>{}, t, valid);
                }
                valid_prev = valid;
            }
            // every LDS access of this step has completed before the next barrier
            wait_lgkm0();
        }

        // ---- segment epilogue: partial statistics at slot w + b
        if (active) {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int j = pbase + 16 * sb + l16;
                const int64_t base = (slot * a.H + head) * a.m + j;
                float z = Zs[sb];
                z += __shfl_xor(z, 16, 64);
                z += __shfl_xor(z, 32, 64);
                if (g == 0) {
                    a.part.M[base] = Mc[sb];
                    a.part.Z[base] = z;
                }
#pragma unroll
                for (int db = 0; db < 2; ++db)
                    __builtin_nontemporal_store(
                        acc[sb][db], (f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH, pbase / 16 + sb, db, lane));
            }
        }
        wait_vm<0>();
        wait_lgkm0();
        block_barrier();
    }
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
