// sa_bf16_stream.hip -- the streaming Sketch Attention forward for bf16 on
// gfx950 (MI355X): the FlashSA computation of section 4.4 of the SequenceO1
// paper -- score blocks, running softmax statistics and aggregation fused,
// the m x n score matrix never leaving registers -- built around the chip's
// direct-to-LDS loads.
//
// Block = one row range (sa_internal.h) x NH heads x (m / 32) prototype
// blocks, one (head, 32-prototype block) unit per wave, NW waves.  Blocks are
// shaped so that every SIMD runs four waves (16 waves and one block per CU,
// or 8 waves and two blocks), and each wave fits in 128 registers: the
// latency of one wave's LDS reads, MFMAs and exps is hidden by the others.
// K and V rows of the block's heads (NH*dh*2 contiguous bytes of every row)
// stream through an LDS ring of kStages 32-row stages:
//   * every stage is filled by global_load_lds_dwordx4 (16 bytes per lane,
//     no registers involved); kStages-1 stages are in flight while one is
//     computed, and each wave waits with a counted s_waitcnt vmcnt for its
//     own part of the stage it needs before the block barrier;
//   * LDS rows are XOR-swizzled per 16-byte chunk: K so that 16-byte MFMA
//     operand reads of consecutive rows hit distinct banks, V (pairs of
//     chunks kept together) so that the ds_read_b64_tr_b16 transposed reads
//     that build the V^T operand do too;
//   * scores S^T = K P^T and the aggregate O^T += V^T p^T run on
//     v_mfma_f32_16x16x32_bf16 (P fragments stay in registers); each lane
//     owns one prototype column, so softmax statistics are lane-local;
//   * history axis: p = 2^(s*c - M) with a lazily moved maximum M (moved only
//     when a lane's tile sum would exceed 2^16), running sum by
//     v_dot2c_f32_bf16 on the same bf16 p the aggregation uses;
//   * rows past the segment end are loaded from a clamped, valid row and
//     masked rows are loaded as they are; both get weight 0 and their V
//     values are zeroed in registers before the aggregation, so neither can
//     leak, NaN included.  A stage's mask bytes (and, on the prototype axis,
//     its rows' normalisers) come into LDS with the stage, by 4-byte
//     direct-to-LDS loads counted with its other loads: plain loads at the
//     point of use would make the compiler, which cannot count the ring's
//     asm loads, wait for all of them, draining the ring once per stage.
#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kStages = 4;   // ring slots: 3 stages in flight, 1 computed

// Ring bytes of a block, and the blocks per CU the 160 KB of LDS allow (at
// most the two that give four waves per SIMD with 8-wave blocks).  dh = 128
// waves need more than 128 registers (their P fragments and sums double), so
// that shape runs one 8-wave block, two waves per SIMD, per CU.
constexpr int ring_bytes(int DH, int NH) { return kStages * 2 * 32 * NH * DH * 2; }
constexpr int blocks_per_cu(int DH, int NW, int NH) {
    return DH == 128 ? 1
                     : (16 / NW) < (160 * 1024 / ring_bytes(DH, NH)) ? (16 / NW) : (160 * 1024 / ring_bytes(DH, NH));
}

}  // namespace

template <int DH, int NW, int NH, int MB, bool MASKED, bool PROTO, bool EXACT>
__global__ __launch_bounds__(NW * 64, NW / 4 * blocks_per_cu(DH, NW, NH)) void sa_bf16_stream_kernel(FwdArgs a,
                                                                                                        int PB) {
    constexpr int S = kStages;
    constexpr int CPR = NH * DH / 8;                      // 16-byte chunks per row per tensor
    constexpr int ROWB = CPR * 16;                        // bytes per row per tensor
    constexpr int D = 32 * CPR / (NW * 64);               // DMA ops per wave per tensor per stage
    constexpr int STAGE = 32 * ROWB;                      // bytes per tensor per stage
    // vector-memory ops per wave per stage: K and V, on the prototype axis one
    // 4-byte load of the rows' normalisers, with a mask one of its bytes
    constexpr int VMS = 2 * D + (PROTO ? 1 : 0) + (MASKED ? 1 : 0);
    constexpr int AHEAD = S - 1;                          // stages issued ahead of the one computed
    constexpr int FK = CPR < 16 ? CPR : 16;               // K swizzle period (rows)
    constexpr int FV = (CPR < 16 ? CPR : 16) / 2;         // V swizzle period (rows), chunk pairs
    constexpr int NSB = MB / 16;
    static_assert(MB == 32, "prototypes per wave");
    constexpr int KC = DH / 32;
    constexpr int DB = DH / 16;
    static_assert(D >= 1 && D * NW * 64 == 32 * CPR, "a stage is whole DMA ops per wave");
    static_assert(CPR >= 4 && CPR <= 32 && (CPR & (CPR - 1)) == 0, "row width");
    static_assert((AHEAD - 1) * VMS < 64, "ring depth");

    __shared__ __attribute__((aligned(1024))) unsigned char ring[S][2][STAGE];
    // prototype axis: each wave's 64 dwords of a stage's per-(row, head)
    // normalisers, entry row * NH + head for the first 32 * NH of them
    __shared__ __attribute__((aligned(16))) float nlring[PROTO ? S : 1][PROTO ? NW * 64 : 1];
    // with a mask: each wave's own copy of a stage's mask bytes, lane i < 32
    // holding the 4-byte word that contains row i's byte
    __shared__ __attribute__((aligned(16))) uint32_t mkring[MASKED ? S : 1][MASKED ? NW * 64 : 1];

    if (offsets_rejected(a.status)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;

    // (row range w, head group gy) of this block.  Blocks are dispatched in
    // linear order and round-robin over the 8 XCDs; with G a multiple of 8
    // the ranges w < G/2 (all head groups) come first, and every head group
    // of range w sits on XCD w % 8 as with the plain (x, y) order.
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

    // block heads and this wave's unit: NH heads x PB prototype blocks = NW,
    // or, when a head has more prototype blocks than the block has waves
    // (PB > NW, then NH = 1), PB / NW blocks per head with NW blocks each
    const int bph = PB > NW ? PB / NW : 1;
    const int h0 = PB > NW ? gy / bph : gy * NH;
    const int hl = PB > NW ? 0 : wave / PB;
    const int head = h0 + hl;
    const int pb = PB > NW ? (gy % bph) * NW + wave : wave % PB;
    const bool active = head < a.H;

    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, a.split);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);

    const bf16* Pg = (const bf16*)a.P;
    const unsigned char* Kg = (const unsigned char*)a.K;
    const unsigned char* Vg = (const unsigned char*)a.V;
    const int hc = min(h0, a.H - 1);       // first head of the block (clamped for idle tails)
    const int64_t krow = a.k_stride * 2, vrow = a.v_stride * 2;   // bytes between rows

    bf16x8 pf[NSB][KC];
    auto load_p = [&](int b) {
        const int hh = active ? head : hc;
        const bf16* base = Pg + (int64_t)b * a.q_batch_stride + ((int64_t)hh * a.m + (active ? pb : 0) * MB) * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 v = *(const bf16x8*)(base + (int64_t)(16 * sb + l16) * DH + 32 * kc + 8 * g);
                if constexpr (PROTO || EXACT) {
                    pf[sb][kc] = v;
                } else {
                    // history axis: scale * log2(e) folded into the prototypes
                    // (rounded to bf16 once), so the products are base-2 scores
                    bf16x8 w;
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const bf16x2 q = pack2((float)v[e] * a.c, (float)v[e + 1] * a.c);
                        w[e] = q[0];
                        w[e + 1] = q[1];
                    }
                    pf[sb][kc] = w;
                }
            }
        // settle the loads here (no ring traffic is in flight yet) so that the
        // compiler does not re-wait for them, and with them for the ring, in the loop
        wait_vm<0>();
    };
    if (a.q_batch_stride == 0) load_p(0);

    // per-lane DMA geometry: op (wave*D + d) writes 1 KB; lane writes 16 B at
    // LDS offset op*1024 + lane*16 = row * ROWB + slot * 16, fetching the
    // global chunk that the swizzle places in that slot
    // (the byte offsets of full stages are computed once; the last stage of a
    // segment clamps rows past its end)
    int dma_row[D];
    uint32_t koff[D], voff[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int off = (wave * D + d) * 1024 + lane * 16;
        dma_row[d] = off / ROWB;
        const int slot = (off % ROWB) / 16;
        koff[d] = (uint32_t)(dma_row[d] * (int)krow + (slot ^ (dma_row[d] % FK)) * 16);
        voff[d] = (uint32_t)(dma_row[d] * (int)vrow + (slot ^ (2 * (dma_row[d] % FV))) * 16);
    }
    // per-lane LDS byte offsets inside one 32-row stage (the swizzle of a row
    // depends on row % 16 only, so both 16-row halves share them)
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0][0];
    const uint32_t nl_lds = (uint32_t)(uintptr_t)(lds_void*)&nlring[0][0];
    const uint32_t mk_lds = (uint32_t)(uintptr_t)(lds_void*)&mkring[0][0];
    // (typed LDS pointers: the slot and half offsets of a stage are then
    // constant indices that fold into the reads' instruction offsets)
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    lds_bf16x8* klane[KC];   // K operand reads, slot 0
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int row = l16, c = hl * (DH / 8) + 4 * kc + g;
        klane[kc] = (lds_bf16x8*)(uintptr_t)(ring_lds + row * ROWB + ((c ^ (row % FK)) * 16));
    }
    lds_i16x4* vlane[DB];   // V^T transposed reads, slot 0
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int kq = l16 >> 2, q = l16 & 3;
        const int row = 4 * g + kq, colb = hl * DH * 2 + (16 * db + 4 * q) * 2;
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
        // segment bases, wave-uniform: moved to scalar registers once, so that
        // the per-stage advance below is scalar arithmetic
        const unsigned char* kseg = uniform_ptr(Kg + gbase * krow + (int64_t)h0 * DH * 2);
        const unsigned char* vseg = uniform_ptr(Vg + gbase * vrow + (int64_t)h0 * DH * 2);

        // ---- issue stage t into ring slot `slot` (t % S; callers pass it as a
        // literal so that every ring address folds into instruction offsets).
        // Every lane of every wave issues; stages are issued in order, so the
        // wave-uniform bases advance by 32 rows per stage (scalar registers);
        // lane offsets are the precomputed ones, clamped in the last stage so
        // that rows past the segment end re-read its last row
        const unsigned char* knext = kseg;
        const unsigned char* vnext = vseg;
        auto issue = [&](int t, int slot) {
            const uint32_t slot_lds = ring_lds + (uint32_t)(slot * 2 * STAGE) + (uint32_t)(wave * D * 1024);
            const int r0 = t * 32;
            const int last = nrows32 - 1 - r0;
            const unsigned char* kb = knext;
            const unsigned char* vb = vnext;
            knext += 32 * krow;
            vnext += 32 * vrow;
            const bool tail = last < 31;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                uint32_t ko = koff[d], vo = voff[d];
                if (tail) {
                    const int over = max(dma_row[d] - last, 0);
                    ko -= (uint32_t)(over * (int)krow);
                    vo -= (uint32_t)(over * (int)vrow);
                }
                dma16s(kb, ko, __builtin_amdgcn_readfirstlane(slot_lds + d * 1024));
                dma16s(vb, vo, __builtin_amdgcn_readfirstlane(slot_lds + STAGE + d * 1024));
            }
            if constexpr (MASKED) {
                // lane -> row (lane % 32) clamped to the segment; the load takes
                // the aligned 4-byte word holding the row's mask byte (it stays
                // in the byte's 4-byte-aligned word, so in the byte's page)
                const uintptr_t m0 = (uintptr_t)(a.mask + gbase + r0);
                const int rr = min(lane & 31, last);
                dma4c((const void*)(m0 & ~(uintptr_t)3), (uint32_t)((int)(m0 & 3) + rr) & ~3u,
                      __builtin_amdgcn_readfirstlane(mk_lds + (uint32_t)((slot * NW + wave) * 256)));
            }
            if constexpr (PROTO) {
                // lane -> entry (wave*64 + lane) mod 32 NH: row e / NH (clamped
                // to the segment), head hc + e % NH; the entries past 32 NH repeat
                const int e = (wave * 64 + lane) % (32 * NH);
                const int rr = min(e / NH, last);
                const float* nb = a.lse2_tok + (gbase + r0) * a.H + hc;
                dma4c(nb, (uint32_t)((rr * a.H + min(e % NH, a.H - 1 - hc)) * 4),
                      __builtin_amdgcn_readfirstlane(nl_lds + (uint32_t)((slot * NW + wave) * 256)));
            }
        };
        // validity bits of stage t (32 rows): rows past the segment end or masked are 0
        auto unit_valid = [&](int t, int slot) -> uint32_t {
            const int64_t r0 = (int64_t)t * 32;
            const int rows_here = (int)min((int64_t)32, nrows - r0);
            bool v = lane < rows_here;
            if constexpr (MASKED) {
                // the stage's mask words arrived with it (this wave's own copy)
                const uint32_t m0 = (uint32_t)((uintptr_t)(a.mask + gbase + r0) & 3);
                const int sh = 8 * (int)((m0 + (uint32_t)min(lane & 31, rows_here - 1)) & 3);
                const uint32_t wd = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                    mk_lds + (uint32_t)((slot * NW + wave) * 256 + 4 * lane));
                v = v && ((wd >> sh) & 0xffu) != 0;
            }
            return (uint32_t)__ballot(v);
        };

        // history axis: the running maximum M of each of the lane's prototypes
        // is kept negated in all four entries of a tuple that is the first
        // score product's accumulator input, so the products come out as
        // s - M and a weight is one exp2 (the tuple changes only when M does).
        // Until the prototype meets a valid row, M is 0 (so the products are
        // the scores themselves) and Zs is -1, which sends every tile to the
        // exact path that sets M from the scores.  With EXACT the prototypes
        // are not pre-scaled: products and M are in units of the raw scores
        // s, a weight is 2^(c (s - M)) and the stored maximum c M.
        float Zs[NSB];
        f32x4 nM[NSB];
        f32x4 acc[NSB][DB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            nM[sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
            Zs[sb] = PROTO ? 0.f : -1.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // one 32-row stage: scores, weights, aggregation
        auto unit = [&](int t, int slot, uint32_t valid) {
            // all 32 rows of the stage are inside the segment (without a mask
            // that is valid == all ones)
            const bool seg_full = MASKED ? (t + 1) * 32 <= nrows32 : valid == 0xffffffffu;
            const uint32_t sbase = (uint32_t)(slot * 2 * STAGE);
            // S^T = K P^T (two 16-row halves)
            f32x4 s[2][NSB];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                lds_bf16x8* p0 = klane[kc] + sbase / 16;
                const bf16x8 k0 = p0[0];
                const bf16x8 k1 = p0[16 * ROWB / 16];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const f32x4 zc = PROTO ? (f32x4){0.f, 0.f, 0.f, 0.f} : nM[sb];
                    const f32x4 z0 = kc == 0 ? zc : s[0][sb];
                    const f32x4 z1 = kc == 0 ? zc : s[1][sb];
                    s[0][sb] = mfma(k0, pf[sb][kc], z0);
                    s[1][sb] = mfma(k1, pf[sb][kc], z1);
                }
            }
            // V^T operands (issued now, used after the weights)
            i16x4 lo[DB], hi[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                lo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vlane[db] + sbase / 8);
                hi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vlane[db] + (sbase + 16 * ROWB) / 8);
            }
            const uint32_t vj = lane_slots(valid, g);
            bf16x8 pk[NSB];
            if constexpr (PROTO) {
                // prototype axis: weights 2^(s*c - lse2[row]) with the per-row normaliser
                // the stage's normalisers arrived with it (direct-to-LDS)
                const uint32_t nls = nl_lds + (uint32_t)(slot * NW * 256);
                float nl[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float v = *(const __attribute__((address_space(3))) float*)(uintptr_t)(
                        nls + (uint32_t)((tok_of(g, j) * NH + hl) * 4));
                    nl[j] = ((vj >> j) & 1) ? v : 0.f;
                }
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    float p[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(fmaf(s[j >> 2][sb][j & 3], a.c, -nl[j])) : 0.f;
                    pk[sb] = cat8(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
                }
            } else {
                // fast path: the running maximum stays, Z += the tile's sum
                float zt[NSB], f[NSB];
                bool fits = true;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    float p[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        p[j] = __builtin_amdgcn_exp2f(EXACT ? s[j >> 2][sb][j & 3] * a.c : s[j >> 2][sb][j & 3]);
                        // with a mask, masked rows get weight 0 here, so they
                        // do not force the exact path (a no-op where the mask
                        // is all ones, which keeps that bitwise equal to no mask)
                        if constexpr (MASKED) p[j] = ((vj >> j) & 1) ? p[j] : 0.f;
                    }
                    const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                    const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                    pk[sb] = cat8(q0, q1, q2, q3);
                    zt[sb] = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
                    f[sb] = 1.f;
                    // false for NaN and Inf too, and before the first valid row
                    fits = fits && (zt[sb] <= kLazyBound) && (Zs[sb] >= 0.f);
                }
                // rare exact path (then-only, so the common path keeps its
                // values in place): validity, running-maximum update, rescale
                if (__builtin_expect(!(__all(fits) && seg_full), 0)) {
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) {
                        // scores relative to 0 again (the tuple held -M; before
                        // the first valid row M = 0 and the products are the scores)
                        const float Mold = -nM[sb][0];
                        const bool none = Zs[sb] < 0.f;         // no valid row met yet
                        float x[8];
                        float tm = -INFINITY;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            x[j] = ((vj >> j) & 1) ? s[j >> 2][sb][j & 3] + Mold : -INFINITY;
                            tm = fmaxf(tm, x[j]);
                        }
                        tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
                        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
                        const float Mnew = none ? tm : fmaxf(Mold, tm);
                        const bool found = Mnew != -INFINITY;   // the prototype has a valid row
                        // (while it has none, M stays 0 and Zs -1)
                        const float Mset = found ? Mnew : 0.f;
                        f[sb] = none ? 0.f
                                     : (Mset == Mold ? 1.f : __builtin_amdgcn_exp2f(EXACT ? (Mold - Mset) * a.c : Mold - Mset));
                        float p[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(EXACT ? (x[j] - Mset) * a.c : x[j] - Mset) : 0.f;
                        const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                        const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                        pk[sb] = cat8(q0, q1, q2, q3);
                        zt[sb] = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
                        if (none && !found) zt[sb] = -1.f;      // Zs = -1 * 0 - 1 keeps the sentinel
                        nM[sb] = (f32x4){-Mset, -Mset, -Mset, -Mset};
#pragma unroll
                        for (int db = 0; db < DB; ++db) acc[sb][db] *= f[sb];
                    }
                }
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) Zs[sb] = fmaf(Zs[sb], f[sb], zt[sb]);
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
        };

        // stage t, in ring slot `slot` (= t % S, a literal at every call)
        auto stage = [&](int t, int slot) {
            // this wave's part of stage t has landed; the barrier makes the
            // stage complete and frees slot (t - 1) % S for stage t + AHEAD
            wait_after<AHEAD - 1, VMS>(min(AHEAD - 1, ntiles - 1 - t));
            block_barrier();
            if (t + AHEAD < ntiles) issue(t + AHEAD, (slot + AHEAD) % S);
            const uint32_t valid = unit_valid(t, slot);
            if (active) unit(t, slot, valid);
            // every LDS read of this stage has completed before the next barrier
            wait_lgkm0();
        };
        static_assert(S == 4, "the stage loop is unrolled by the ring size");
        if (0 < ntiles) issue(0, 0);
        if (1 < ntiles) issue(1, 1);
        if (2 < ntiles) issue(2, 2);
        int t = 0;
        for (; t + S <= ntiles; t += S) {
            stage(t, 0);
            stage(t + 1, 1);
            stage(t + 2, 2);
            stage(t + 3, 3);
        }
        if (t < ntiles) stage(t, 0);
        if (t + 1 < ntiles) stage(t + 1, 1);
        if (t + 2 < ntiles) stage(t + 2, 2);

        // ---- segment epilogue: partial statistics at slot w + b (the sums in
        // lane order, 1 KB per store, written through to memory: these writes
        // are the kernel's tail, and lines left dirty in the caches would be
        // written back during the next launch's reads, ~1 % slower)
        if (active) {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int j = pb * MB + 16 * sb + l16;
                const int64_t base = (slot * a.H + head) * a.m + j;
                if constexpr (!PROTO) {
                    float z = fmaxf(Zs[sb], 0.f);     // the -1 of a prototype with no valid row
                    z += __shfl_xor(z, 16, 64);
                    z += __shfl_xor(z, 32, 64);
                    if (g == 0) {
                        // no valid row in the segment: M = -inf, as the merge expects
                        a.part.M[base] = z > 0.f ? (EXACT ? -nM[sb][0] * a.c : -nM[sb][0]) : -INFINITY;
                        a.part.Z[base] = z;
                    }
                }
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    store16_wt((f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH, (pb * MB) / 16 + sb, db, lane),
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

namespace {

template <int DH, int NW, int NH, int MB>
hipError_t launch_stream(const FwdArgs& a, bool masked, int PB, hipStream_t s) {
    dim3 grid(a.G, PB > NW ? a.H * (PB / NW) : a.H / NH), block(NW * 64);
    const bool proto = a.norm == 1, exact = !proto && a.exact_scale;
#define SA_LAUNCH(M_, P_, E_) \
    hipLaunchKernelGGL((sa_bf16_stream_kernel<DH, NW, NH, MB, M_, P_, E_>), grid, block, 0, s, a, PB)
    if (proto) {
        if (masked) SA_LAUNCH(true, true, false);
        else SA_LAUNCH(false, true, false);
    } else if constexpr (DH == 128) {
        // the history axis at this width runs sa_bf16_stream_d128_kernel
        return hipErrorInvalidValue;
    } else if (exact) {
        if (masked) SA_LAUNCH(true, false, true);
        else SA_LAUNCH(false, false, true);
    } else {
        if (masked) SA_LAUNCH(true, false, false);
        else SA_LAUNCH(false, false, false);
    }
#undef SA_LAUNCH
    return hipGetLastError();
}

// Compiled block shapes (dh, waves, heads per block): each stage of 32 rows x
// NH*dh*2 bytes is whole 1 KB DMA ops per wave, rows are at most 512 bytes.
struct Shape {
    int dh, NW, NH, MB;
};
constexpr Shape kShapes[] = {{64, 16, 4, 32}, {64, 8, 2, 32}, {64, 8, 4, 32}, {32, 16, 8, 32},
                             {32, 8, 4, 32},  {32, 8, 8, 32}, {128, 8, 1, 32}};

}  // namespace

// Streaming kernel shapes: dh in {32, 64}, m a multiple of 32, a compiled
// (NW, NH) with NW = NH * m / 32 (one wave per (head, 32-prototype) unit) and
// H a multiple of NH.  Preference: 8 waves (two blocks per CU, four waves per
// SIMD, independent barriers), then 16 waves (one block per CU);
// prefer_nw = 16 reverses the order.
bool stream_config(int dh, int m, int H, int prefer_nw, StreamConfig* cfg) {
    if (dh == 128) {
        // one head per block, 8 waves = 256 prototypes; m / 256 blocks per head
        if (m % 256 != 0) return false;
        cfg->PB = m / 32;
        cfg->MB = 32;
        cfg->NH = 1;
        cfg->NW = 8;
        cfg->groups = H * (m / 256);
        cfg->blocks_per_cu = blocks_per_cu(128, 8, 1);
        return true;
    }
    if (!(dh == 32 || dh == 64) || m % 32 != 0) return false;
    const int prefer = prefer_nw == 16 ? 16 : 8;
    const int MB = 32, PB = m / MB;
    for (int pass = 0; pass < 2; ++pass) {
        const int NW = pass == 0 ? prefer : 24 - prefer;
        for (const Shape& sh : kShapes) {
            if (sh.dh != dh || sh.NW != NW || sh.MB != MB || sh.NH * PB != NW || H % sh.NH != 0) continue;
            cfg->PB = PB;
            cfg->MB = MB;
            cfg->NH = sh.NH;
            cfg->NW = NW;
            cfg->groups = H / sh.NH;
            cfg->blocks_per_cu = blocks_per_cu(dh, NW, sh.NH);
            return true;
        }
    }
    return false;
}

hipError_t launch_bf16_stream(const FwdArgs& a, const StreamConfig& cfg, hipStream_t s) {
    const bool masked = a.mask != nullptr;
    const int dh = a.dh, NH = cfg.NH, PB = cfg.PB, NW = cfg.NW, MB = cfg.MB;
#define SA_STREAM(D_, W_, N_, M_) \
    if (dh == D_ && NW == W_ && NH == N_ && MB == M_) return launch_stream<D_, W_, N_, M_>(a, masked, PB, s);
    SA_STREAM(64, 16, 4, 32) SA_STREAM(64, 8, 2, 32) SA_STREAM(64, 8, 4, 32) SA_STREAM(32, 16, 8, 32)
    SA_STREAM(32, 8, 4, 32) SA_STREAM(32, 8, 8, 32) SA_STREAM(128, 8, 1, 32)
#undef SA_STREAM
    return hipErrorInvalidValue;
}

}  // namespace sa
