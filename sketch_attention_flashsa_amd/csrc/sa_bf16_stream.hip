// sa_bf16_stream.hip -- the streaming Sketch Attention forward for bf16 on
// gfx950 (MI355X): the FlashSA computation of section 4.4 of the SequenceO1
// paper -- score blocks, running softmax statistics and aggregation fused,
// the m x n score matrix never leaving registers -- built around the chip's
// direct-to-LDS loads.
//
// Block = one row range (sa_internal.h) x NH heads x (m / MB) prototype
// blocks, one (head, MB-prototype block) unit per wave.  K and V rows of the
// block's heads stream through an LDS ring of kStages stages:
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
//     leak, NaN included.  The mask bytes of a stage are read when the stage
//     is consumed (a plain load the compiler waits for), so masked inputs
//     keep less of the ring in flight than unmasked ones.
#include <stdlib.h>
#include <string.h>

#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kStages = 4;   // ring slots: 2 stages in flight, 1 computed, 1 still read for V

}  // namespace

template <int DH, int MB, int NW, int NH, bool MASKED, bool PROTO, int S = kStages, int WPE = 2, int DMUL = 1>
__global__ __launch_bounds__(NW * 64, WPE) void sa_bf16_stream_kernel(FwdArgs a, int PB) {
    constexpr int CPR = NH * DH / 8;                      // 16-byte chunks per row per tensor
    constexpr int ROWB = CPR * 16;                        // bytes per row per tensor
    constexpr int D = DMUL * ((32 * CPR + NW * 64 - 1) / (NW * 64));  // DMA ops per wave per tensor per stage
    constexpr int TR = NW * D * 64 / CPR;                 // rows per stage
    constexpr int NSUB = TR / 32;                         // 32-row units per stage
    constexpr int STAGE = TR * ROWB;                      // bytes per tensor per stage
    constexpr int VMS = 2 * D;                            // vector-memory ops per wave per stage
    constexpr int AHEAD = S - 2;                          // stages issued ahead of the one computed
    constexpr int FK = CPR < 16 ? CPR : 16;               // K swizzle period (rows)
    constexpr int FV = (CPR < 16 ? CPR : 16) / 2;         // V swizzle period (rows), chunk pairs
    constexpr int NSB = MB / 16;
    constexpr int KC = DH / 32;
    constexpr int DB = DH / 16;
    static_assert(TR % 32 == 0 && TR <= 128, "stage rows");
    static_assert(CPR >= 4 && CPR <= 64 && (CPR & (CPR - 1)) == 0, "row width");
    static_assert(NW * D * 1024 == STAGE, "stage = whole DMA ops");
    static_assert(S >= 3 && S <= 8 && (AHEAD - 1) * VMS < 64, "ring depth");

    __shared__ __attribute__((aligned(1024))) unsigned char ring[S][2][STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int w = blockIdx.x;

    // block heads and this wave's unit
    const int units_per_block = NH * PB < NW ? NH * PB : NW;
    const int blocks_per_head = PB > NW ? PB / NW : 1;
    const int h0 = (PB > NW) ? blockIdx.y / blocks_per_head : blockIdx.y * NH;
    const int pb0 = (PB > NW) ? (blockIdx.y % blocks_per_head) * NW : 0;
    const int hl = (PB > NW) ? 0 : wave / PB;
    const int head = h0 + hl;
    const int pb = (PB > NW) ? pb0 + wave : wave % PB;
    const bool active = wave < units_per_block && head < a.H;

    const int64_t total = a.users.total();
    const int64_t R = chunk_rows(total, a.G, a.R_fixed, a.R_min);
    const int64_t v_lo = (int64_t)w * R;
    if (v_lo >= total) return;
    const int64_t v_hi = min(v_lo + R, total);

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
            for (int kc = 0; kc < KC; ++kc)
                pf[sb][kc] = *(const bf16x8*)(base + (int64_t)(16 * sb + l16) * DH + 32 * kc + 8 * g);
        // settle the loads here (no ring traffic is in flight yet) so that the
        // compiler does not re-wait for them, and with them for the ring, in the loop
        wait_vm<0>();
    };
    if (a.q_batch_stride == 0) load_p(0);

    // per-lane DMA geometry: op (wave*D + d) writes 1 KB; lane writes 16 B at
    // LDS offset op*1024 + lane*16 = row * ROWB + slot * 16, fetching the global
    // chunk that the swizzle places in that slot
    int dma_row[D], dma_ck[D], dma_cv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int off = (wave * D + d) * 1024 + lane * 16;
        dma_row[d] = off / ROWB;
        const int slot = (off % ROWB) / 16;
        dma_ck[d] = (slot ^ (dma_row[d] % FK)) * 16;
        dma_cv[d] = (slot ^ (2 * (dma_row[d] % FV))) * 16;
    }
    // per-lane LDS byte offsets inside one 32-row unit (the swizzle of a row
    // depends on row % 16 only, so every unit and both 16-row halves share them)
    int koff[KC], voff[DB];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int row = l16, c = hl * (DH / 8) + 4 * kc + g;
        koff[kc] = row * ROWB + ((c ^ (row % FK)) * 16);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int kq = l16 >> 2, q = l16 & 3;
        const int row = 4 * g + kq, colb = hl * DH * 2 + (16 * db + 4 * q) * 2;
        voff[db] = row * ROWB + (((colb >> 4) ^ (2 * (row % FV))) * 16) + (colb & 15);
    }
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0][0];
    uint32_t vlane[DB];   // LDS address of this lane's V^T reads in slot 0, unit 0
#pragma unroll
    for (int db = 0; db < DB; ++db) vlane[db] = ring_lds + STAGE + voff[db];
    uint32_t klane[KC];   // LDS address of this lane's K reads in slot 0, unit 0
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) klane[kc] = ring_lds + koff[kc];

    int b = a.users.find(v_lo);
    for (; b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        if (a.q_batch_stride != 0) load_p(b);
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int64_t nrows = s_hi - s_lo;
        const int ntiles = (int)((nrows + TR - 1) / TR);
        const int nunits = (int)((nrows + 31) / 32);
        const unsigned char* kseg = Kg + gbase * krow + (int64_t)h0 * DH * 2;
        const unsigned char* vseg = Vg + gbase * vrow + (int64_t)h0 * DH * 2;
        // this lane's source addresses: running pointers advanced one stage per
        // issue, and the segment's last row (rows past the end re-read it)
        const unsigned char* kp[D];
        const unsigned char* vp[D];
        const unsigned char* klast[D];
        const unsigned char* vlast[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            kp[d] = kseg + dma_row[d] * krow + dma_ck[d];
            vp[d] = vseg + dma_row[d] * vrow + dma_cv[d];
            klast[d] = kseg + (nrows - 1) * krow + dma_ck[d];
            vlast[d] = vseg + (nrows - 1) * vrow + dma_cv[d];
        }
        const int64_t kstep = TR * krow, vstep = TR * vrow;
        const int nrows32 = (int)nrows;

        // ---- issue stage t into ring slot t % S (every lane of every wave, always);
        // stages are issued in order, so t == (number issued so far)
        auto issue = [&](int t) {
            const uint32_t slot_lds = ring_lds + (uint32_t)((t % S) * 2 * STAGE) + (uint32_t)(wave * D * 1024);
            const int r0 = t * TR;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const bool in = r0 + dma_row[d] < nrows32;
                dma16(in ? kp[d] : klast[d], __builtin_amdgcn_readfirstlane(slot_lds + d * 1024));
                dma16(in ? vp[d] : vlast[d], __builtin_amdgcn_readfirstlane(slot_lds + STAGE + d * 1024));
                kp[d] += kstep;
                vp[d] += vstep;
            }
        };
        // validity bits of unit u (32 rows): rows past the segment end or masked are 0
        auto unit_valid = [&](int u) -> uint32_t {
            const int64_t r0 = (int64_t)u * 32;
            const int rows_here = (int)min((int64_t)32, nrows - r0);
            bool v = lane < rows_here;
            if constexpr (MASKED) v = v && a.mask[gbase + r0 + min(lane, rows_here - 1)] != 0;
            return (uint32_t)__ballot(v);
        };
        // S^T = K P^T for unit u
        auto scores = [&](int u, f32x4 (&s)[2][NSB]) {
            const uint32_t kb = (uint32_t)(((u / NSUB) % S) * 2 * STAGE + (u % NSUB) * 32 * ROWB);
            uint32_t addr[KC];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) addr[kc] = klane[kc] + kb;
            bf16x8 ka[2][KC];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const __attribute__((address_space(3))) bf16x8* pk0 =
                    (const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr[kc];
                ka[0][kc] = pk0[0];
                ka[1][kc] = pk0[16 * ROWB / 16];
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    f32x4 d = mfma(ka[st][0], pf[sb][0], (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int kc = 1; kc < KC; ++kc) d = mfma(ka[st][kc], pf[sb][kc], d);
                    s[st][sb] = d;
                }
            }
        };

        float Mc[NSB], Zs[NSB];
        f32x4 acc[NSB][DB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            Mc[sb] = -INFINITY;
            Zs[sb] = 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // fast-path weights of a unit (history axis): p = 2^(s*c - M); returns
        // whether every lane's tile sum stayed within the lazy bound
        auto weights_fast = [&](const f32x4 (&s)[2][NSB], bf16x8 (&pk)[NSB], float (&zt)[NSB]) -> bool {
            bool fits = true;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const float nm = -Mc[sb];
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[j >> 2][sb][j & 3], a.c, nm));
                const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                pk[sb] = cat8(q0, q1, q2, q3);
                zt[sb] = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
                fits = fits && (zt[sb] <= kLazyBound);    // false for NaN and Inf too
            }
            return fits;
        };
        // exact weights: validity, running-maximum update and rescale.  It
        // overwrites the fast path's pk and zt (the tile sums) and sets the
        // rescale factors f; the caller applies Z = Z f + zt.
        auto weights_exact = [&](const f32x4 (&s)[2][NSB], uint32_t valid, bf16x8 (&pk)[NSB], float (&zt)[NSB],
                                 float (&f)[NSB]) {
            const uint32_t vj = lane_slots(valid, g);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                float x[8];
                float tm = -INFINITY;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    x[j] = ((vj >> j) & 1) ? s[j >> 2][sb][j & 3] * a.c : -INFINITY;
                    tm = fmaxf(tm, x[j]);
                }
                tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
                tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
                const float Mold = Mc[sb];
                const float Mnew = fmaxf(Mold, tm);
                f[sb] = (Mnew == Mold) ? 1.f : __builtin_amdgcn_exp2f(Mold - Mnew);
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(x[j] - Mnew) : 0.f;
                const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                pk[sb] = cat8(q0, q1, q2, q3);
                zt[sb] = dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
                Mc[sb] = Mnew;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[sb][db] *= f[sb];
            }
        };
        // prototype axis: weights 2^(s*c - lse2[row]) with the per-row normaliser
        auto weights_proto = [&](const f32x4 (&s)[2][NSB], int u, uint32_t valid, bf16x8 (&pk)[NSB]) {
            const uint32_t vj = lane_slots(valid, g);
            float nl[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                nl[j] = ((vj >> j) & 1) ? a.lse2_tok[(gbase + (int64_t)u * 32 + tok_of(g, j)) * a.H + head] : 0.f;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    p[j] = ((vj >> j) & 1) ? __builtin_amdgcn_exp2f(fmaf(s[j >> 2][sb][j & 3], a.c, -nl[j])) : 0.f;
                pk[sb] = cat8(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
            }
        };
        // O^T += V^T p^T for unit u
        auto aggregate = [&](int u, uint32_t valid, const bf16x8 (&pk)[NSB]) {
            const uint32_t vb = (uint32_t)(((u / NSUB) % S) * 2 * STAGE + (u % NSUB) * 32 * ROWB);
            uint32_t addr[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) addr[db] = vlane[db] + vb;
            i16x4 lo[DB], hi[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                lo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr[db]);
                hi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(addr[db] + 16 * ROWB));
            }
            if (valid != 0xffffffffu) {
                // rows outside the segment or masked: zero their values (NaN must not leak)
                const uint32_t vj = lane_slots(valid, g);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (!((vj >> j) & 1)) lo[db][j] = 0;
                        if (!((vj >> (4 + j)) & 1)) hi[db][j] = 0;
                    }
                }
            }
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
        // weights of unit u (held in s, validity in valid), then its aggregation.
        // The exact path is a then-only branch that overwrites the fast path's
        // values in place, so the common path carries no register copies.
        auto finish_unit = [&](int u, const f32x4 (&s)[2][NSB], uint32_t valid, bf16x8 (&pk)[NSB], float (&zt)[NSB],
                               bool fits) {
            if constexpr (PROTO) {
                weights_proto(s, u, valid, pk);
            } else {
                float f[NSB];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) f[sb] = 1.f;
                if (__builtin_expect(!(__all(fits) && valid == 0xffffffffu), 0)) weights_exact(s, valid, pk, zt, f);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) Zs[sb] = fmaf(Zs[sb], f[sb], zt[sb]);
            }
            aggregate(u, valid, pk);
        };
        // wait until this wave's part of stage t has landed, then sync the block
        auto stage_ready = [&](int t) {
            wait_after<AHEAD - 1, VMS>(min(AHEAD - 1, ntiles - 1 - t));
            wait_lgkm0();
            block_barrier();
            if (t + AHEAD < ntiles) issue(t + AHEAD);
        };

#pragma unroll
        for (int t = 0; t < AHEAD; ++t)
            if (t < ntiles) issue(t);

        // software pipeline over 32-row units: step u computes the scores of
        // unit u next to the weights of unit u-1, then aggregates unit u-1.
        // Unrolled by two so the score buffers alternate without copies.
        auto step = [&](int u, f32x4 (&s_cur)[2][NSB], const f32x4 (&s_prev)[2][NSB], uint32_t& valid_prev) {
            if (u % NSUB == 0) stage_ready(u / NSUB);
            const uint32_t valid_cur = unit_valid(u);
            if (active) {
                bf16x8 pk[NSB];
                float zt[NSB];
                bool fits = true;
                scores(u, s_cur);
                if constexpr (!PROTO) fits = weights_fast(s_prev, pk, zt);
                finish_unit(u - 1, s_prev, valid_prev, pk, zt, fits);
            }
            valid_prev = valid_cur;
        };
        auto drain = [&](const f32x4 (&s_last)[2][NSB], uint32_t valid_last) {
            if (active) {
                bf16x8 pk[NSB];
                float zt[NSB];
                bool fits = true;
                if constexpr (!PROTO) fits = weights_fast(s_last, pk, zt);
                finish_unit(nunits - 1, s_last, valid_last, pk, zt, fits);
            }
        };
        f32x4 sA[2][NSB], sB[2][NSB];
        stage_ready(0);
        uint32_t valid_prev = unit_valid(0);
        if (active) scores(0, sA);
        int u = 1;
        for (; u + 1 < nunits; u += 2) {
            step(u, sB, sA, valid_prev);
            step(u + 1, sA, sB, valid_prev);
        }
        if (u < nunits) {
            step(u, sB, sA, valid_prev);
            drain(sB, valid_prev);
        } else {
            drain(sA, valid_prev);
        }

        // ---- segment epilogue: partial statistics at slot w + b
        if (active) {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int j = pb * MB + 16 * sb + l16;
                const int64_t base = (slot * a.H + head) * a.m + j;
                if constexpr (!PROTO) {
                    float z = Zs[sb];
                    z += __shfl_xor(z, 16, 64);
                    z += __shfl_xor(z, 32, 64);
                    if (g == 0) {
                        a.part.M[base] = Mc[sb];
                        a.part.Z[base] = z;
                    }
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) *(f32x4*)(a.part.acc + base * DH + 16 * db + 4 * g) = acc[sb][db];
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

// Ring shape: kStages slots of 32*kStageMul rows (history axis, no mask).
// SA_STREAM_RING="S,MUL" selects another of the compiled shapes (tuning).
template <int DH, int MB, int NW, int NH, int S, int MUL>
void launch_hist(dim3 grid, dim3 block, const FwdArgs& a, int PB, hipStream_t s) {
    hipLaunchKernelGGL((sa_bf16_stream_kernel<DH, MB, NW, NH, false, false, S, 2, MUL>), grid, block, 0, s, a, PB);
}

template <int DH, int MB, int NW, int NH>
hipError_t launch_stream(const FwdArgs& a, bool masked, int PB, hipStream_t s) {
    int groups;
    if (PB > NW) groups = a.H * (PB / NW);
    else groups = (a.H + NH - 1) / NH;
    dim3 grid(a.G, groups), block(NW * 64);
    const bool proto = a.norm == 1;
    if (!masked && !proto) {
        // 64-row stages when a stage of 32 rows is a single DMA op per wave and
        // the ring still fits the LDS; else 32-row stages
        constexpr int CPR = NH * DH / 8;
        constexpr int D1 = (32 * CPR + NW * 64 - 1) / (NW * 64);
        constexpr int TR1 = NW * D1 * 64 / CPR;              // stage rows at MUL = 1
        constexpr int SLOT = 2 * NW * D1 * 1024;             // bytes per slot at MUL = 1
        constexpr bool wide = D1 == 1 && TR1 == 32 && 4 * 2 * SLOT <= 160 * 1024;
        int S = 4, mul = wide ? 2 : 1;
        if (const char* e = getenv("SA_STREAM_RING")) {
            int es = 0, em = 0;
            if (sscanf(e, "%d,%d", &es, &em) == 2) {
                S = es;
                mul = em;
            }
        }
        if (S == 3 && mul == 1) launch_hist<DH, MB, NW, NH, 3, 1>(grid, block, a, PB, s);
        else if (S == 5 && mul == 1 && 5 * SLOT <= 160 * 1024) launch_hist<DH, MB, NW, NH, 5, 1>(grid, block, a, PB, s);
        else if (mul == 2 && wide && S == 3) launch_hist<DH, MB, NW, NH, 3, (wide ? 2 : 1)>(grid, block, a, PB, s);
        else if (mul == 2 && wide) launch_hist<DH, MB, NW, NH, 4, (wide ? 2 : 1)>(grid, block, a, PB, s);
        else launch_hist<DH, MB, NW, NH, 4, 1>(grid, block, a, PB, s);
        return hipGetLastError();
    }
    if (masked && !proto) hipLaunchKernelGGL((sa_bf16_stream_kernel<DH, MB, NW, NH, true, false>), grid, block, 0, s, a, PB);
    if (!masked && proto) hipLaunchKernelGGL((sa_bf16_stream_kernel<DH, MB, NW, NH, false, true>), grid, block, 0, s, a, PB);
    if (masked && proto) hipLaunchKernelGGL((sa_bf16_stream_kernel<DH, MB, NW, NH, true, true>), grid, block, 0, s, a, PB);
    return hipGetLastError();
}

}  // namespace

// Streaming kernel shapes: 32 prototypes per wave, NW = 8 (default) or 4
// waves per block; a block covers NH = NW / (m/32) heads (m <= 32*NW) or NW
// of one head's prototype blocks.  SA_STREAM_NW=4 selects 4-wave blocks.
bool stream_config(int dh, int m, int H, StreamConfig* cfg) {
    if (!(dh == 32 || dh == 64) || m % 32 != 0) return false;
    int NW = 8;
    if (const char* e = getenv("SA_STREAM_NW")) NW = atoi(e) == 4 ? 4 : 8;
    const int PB = m / 32;
    int NH;
    if (PB <= NW) {
        if (NW % PB != 0) return false;
        NH = NW / PB;
        if (H % NH != 0) return false;   // a block always stages NH whole heads
    } else {
        if (PB % NW != 0) return false;
        NH = 1;
    }
    if (NH * dh * 2 < 64 || NH * dh > 256) return false;   // row width 64 B .. 512 B per tensor
    if (NW == 4 && NH * dh * 2 < 128) return false;          // keep stages of whole DMA ops
    cfg->PB = PB;
    cfg->NH = NH;
    cfg->NW = NW;
    cfg->groups = (PB > NW) ? H * (PB / NW) : H / NH;
    cfg->blocks_per_cu = NW == 8 ? 1 : 2;
    return true;
}

hipError_t launch_bf16_stream(const FwdArgs& a, const StreamConfig& cfg, hipStream_t s) {
    const bool masked = a.mask != nullptr;
    const int dh = a.dh, NH = cfg.NH, PB = cfg.PB;
    if (cfg.NW == 8) {
#define SA_STREAM(D_, N_) \
    if (dh == D_ && NH == N_) return launch_stream<D_, 32, 8, N_>(a, masked, PB, s);
        SA_STREAM(32, 1) SA_STREAM(32, 2) SA_STREAM(32, 4) SA_STREAM(32, 8)
        SA_STREAM(64, 1) SA_STREAM(64, 2) SA_STREAM(64, 4)
#undef SA_STREAM
    } else {
#define SA_STREAM4(D_, N_) \
    if (dh == D_ && NH == N_) return launch_stream<D_, 32, 4, N_>(a, masked, PB, s);
        SA_STREAM4(32, 2) SA_STREAM4(32, 4) SA_STREAM4(64, 1) SA_STREAM4(64, 2) SA_STREAM4(64, 4)
#undef SA_STREAM4
    }
    return hipErrorInvalidValue;
}

}  // namespace sa
