// sa_proto_stream.hip -- the prototype-axis Sketch Attention forward for bf16
// in one pass over K and V: the normalisation display of section 3.1 of the
// SequenceO1 paper (every history row is spread over the m prototypes of its
// head), with the score, the per-row normaliser and the aggregation fused as
// section 4.4 (FlashSA) describes for the history axis.
//
//   A[j,i] = 2^(s[j,i] c) / Z_i,   Z_i = sum_j 2^(s[j,i] c),   S_j = sum_i A[j,i] V_i
//
// with s = P K^T and c = scale * log2(e).  Block shape, row ranges, DMA ring
// and swizzles are those of the history-axis streaming kernel
// (sa_bf16_stream.hip): NH heads x m/32 prototype blocks, one (head,
// 32-prototype) unit per wave, so a block holds all m prototypes of its heads
// and every row's normaliser is finished inside the block.  Per 32-row stage:
//   * scores S = P K^T on v_mfma_f32_16x16x32_bf16 (P fragments as the A
//     operand; pre-scaled by c unless the row normalisers are written out),
//     so a lane holds 8 prototypes of each of two rows (row l16 of
//     both 16-row halves): the wave's partial row sums of 2^(s c) are seven
//     adds per row, then two lane-row swaps (v_permlane16/32_swap);
//   * the PB waves of a head exchange their partial sums through LDS (a
//     second block barrier per stage) and sum them in a fixed order, so the
//     result does not depend on timing;
//   * while every valid row's partial sum lies in [2^-60, 2^60] the weights
//     are the exponentials 2^(s c) times 1 / Z; otherwise (scores of extreme
//     scale, NaN or Inf) the whole block takes an exact path for the stage:
//     row maxima exchanged first, then sums of 2^(s c - max), as the oracle's
//     definition reads;
//   * the bf16 weights are transposed through a per-wave LDS tile
//     (ds_read_b64_tr_b16) into the aggregation's B operand, and
//     O^T += V^T p^T runs on MFMA as in the history kernel.
// The merge adds the segments' sums in ascending order (sa_merge.hip).
#include "sa_device.h"
#include "sa_proto.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kPStages = 4;            // ring slots, as the history kernel
constexpr int kTileRow = 32;           // bytes per row of a transposition tile (16 bf16)
constexpr float kFitLo = 0x1p-60f;     // fast path: partial row sums inside [2^-60, 2^60]
constexpr float kFitHi = 0x1p60f;

typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int proto_ring_bytes(int DH, int NH) { return kPStages * 2 * 32 * NH * DH * 2; }
constexpr int proto_lds_bytes(int DH, int NW, int NH, bool masked) {
    return proto_ring_bytes(DH, NH) + (masked ? kPStages * 256 : 0) + NW * 32 * kTileRow + 2 * NW * 32 * 4 + 16;
}
// blocks per CU: as the history kernel (the ring decides; at most four waves per SIMD)
constexpr int proto_blocks_per_cu(int DH, int NW, int NH) {
    return (16 / NW) < (160 * 1024 / proto_ring_bytes(DH, NH)) ? (16 / NW) : (160 * 1024 / proto_ring_bytes(DH, NH));
}

// Row sums over the four 16-lane rows g of a wave: z0 is lane (g, l16)'s
// value for row l16 (first 16-row half), z1 for row 16 + l16.  Returns, in
// lanes of even g, the sum of z0 over g, in lanes of odd g the sum of z1
// (permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second; permlane32_swap the upper 32 lanes of the
// first with the lower 32 of the second).  Fixed order, so every lane that
// holds a row's total holds the same bits.
__device__ __forceinline__ float rows_sum(float z0, float z1) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(z0), __float_as_uint(z1), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float z0, float z1) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(z0), __float_as_uint(z1), false, false);
    const float s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace

template <int DH, int NW, int NH, bool MASKED, bool LSE>
__global__ __launch_bounds__(NW * 64, NW / 4 * proto_blocks_per_cu(DH, NW, NH)) void sa_proto_stream_kernel(
    FwdArgs a, float* lse_out) {
    constexpr int S = kPStages;
    constexpr int PB = NW / NH;                            // 32-prototype blocks per head: m = 32 PB
    constexpr int CPR = NH * DH / 8;                       // 16-byte chunks per row per tensor
    constexpr int ROWB = CPR * 16;                         // bytes per row per tensor
    constexpr int D = 32 * CPR / (NW * 64);                // DMA ops per wave per tensor per stage
    constexpr int STAGE = 32 * ROWB;                       // bytes per tensor per stage
    constexpr int VMS = 2 * D + (MASKED ? 1 : 0);          // vector-memory ops per wave per stage
    constexpr int AHEAD = S - 1;
    constexpr int FK = CPR < 16 ? CPR : 16;
    constexpr int FV = (CPR < 16 ? CPR : 16) / 2;
    constexpr int NSB = 2;                                 // 16-prototype blocks per wave
    constexpr int KC = DH / 32;
    constexpr int DB = DH / 16;
    static_assert(PB * NH == NW && PB >= 1, "a block holds all prototypes of its heads");
    static_assert(D >= 1 && D * NW * 64 == 32 * CPR, "a stage is whole DMA ops per wave");
    static_assert(CPR >= 4 && CPR <= 32 && (CPR & (CPR - 1)) == 0, "row width");
    static_assert((AHEAD - 1) * VMS < 64, "ring depth");
    static_assert(proto_lds_bytes(DH, NW, NH, MASKED) * proto_blocks_per_cu(DH, NW, NH) <= 160 * 1024,
                  "the history kernel's blocks per CU still fit");

    __shared__ __attribute__((aligned(1024))) unsigned char ring[S][2][STAGE];
    // with a mask: a stage's mask words, lane i < 32 holding the 4-byte word
    // that contains row i's byte (every wave loads the same words here)
    __shared__ __attribute__((aligned(16))) uint32_t mkring[MASKED ? S : 1][64];
    // per wave: one 32-row x 16-prototype bf16 tile of weights being transposed
    __shared__ __attribute__((aligned(16))) unsigned char ptile[NW][32 * kTileRow];
    // per (stage parity, head, prototype block, row): partial row sums (a
    // stage's are written one loop step before they are read), and maxima
    // on the exact path
    __shared__ __attribute__((aligned(16))) float xsum[2][NH][PB][32];
    __shared__ __attribute__((aligned(16))) float xmax[NH][PB][32];
    // per stage (t & 3): some wave of the block needs the exact path
    __shared__ uint32_t xflag[4];

    if (offsets_rejected(a.status)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;

    // (row range w, head group gy): the history kernel's order
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
    const int hl = wave / PB, pbi = wave % PB;
    const int h0 = gy * NH, head = h0 + hl;               // H is a multiple of NH

    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, a.split);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);

    const unsigned char* Kg = (const unsigned char*)a.K;
    const unsigned char* Vg = (const unsigned char*)a.V;
    const int64_t krow = a.k_stride * 2, vrow = a.v_stride * 2;

    // P fragments as the score product's A operand: lane (g, l16) holds
    // prototype 32 pbi + 16 sb + l16, channels 32 kc + 8 g .. + 7.  Without
    // the lse output they are pre-scaled by c (rounded to bf16 once, as on
    // the history axis: the rounding shifts a row's scores by amounts that
    // mostly cancel in its normalisation), so the products are base-2 scores;
    // the row normaliser itself would keep that shift, so the instance that
    // writes it keeps P exact and scales each product.
    constexpr bool PRESCALE = !LSE;
    bf16x8 pf[NSB][KC];
    {
        const bf16* base = (const bf16*)a.P + ((int64_t)head * a.m + pbi * 32) * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 v = *(const bf16x8*)(base + (int64_t)(16 * sb + l16) * DH + 32 * kc + 8 * g);
                if constexpr (PRESCALE) {
                    bf16x8 w;
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const bf16x2 q = pack2((float)v[e] * a.c, (float)v[e + 1] * a.c);
                        w[e] = q[0];
                        w[e + 1] = q[1];
                    }
                    pf[sb][kc] = w;
                } else {
                    pf[sb][kc] = v;
                }
            }
        wait_vm<0>();
    }
    const float cs = PRESCALE ? 1.f : a.c;   // what the products still need

    // DMA geometry (as the history kernel)
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
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0][0];
    const uint32_t mk_lds = (uint32_t)(uintptr_t)(lds_void*)&mkring[0][0];
    // K fragments as the B operand: row l16 of a half, channels 32 kc + 8 g
    lds_bf16x8* klane[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int row = l16, c = hl * (DH / 8) + 4 * kc + g;
        klane[kc] = (lds_bf16x8*)(uintptr_t)(ring_lds + row * ROWB + ((c ^ (row % FK)) * 16));
    }
    lds_i16x4* vlane[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int kq = l16 >> 2, q = l16 & 3;
        const int row = 4 * g + kq, colb = hl * DH * 2 + (16 * db + 4 * q) * 2;
        vlane[db] = (lds_i16x4*)(uintptr_t)(ring_lds + STAGE + row * ROWB + (((colb >> 4) ^ (2 * (row % FV))) * 16) +
                                            (colb & 15));
    }
    // transposition tile: lane (g, l16) writes the 4 weights of prototypes
    // 4g..4g+3 of row 16 half + l16, and reads back (transposed) prototype
    // l16 of rows 16 half + 4g .. + 3, the B operand's k-slots.  The 8-byte
    // chunk c of row r sits at chunk c ^ ((r >> 2) & 3): the rows that share
    // banks (4 apart with 32-byte rows) then hold different chunks, so each
    // 16-lane pass of the writes (16 rows, one chunk each) and of the
    // transposed reads (4 rows x 4 chunks) touches distinct banks
    const uint32_t tile = (uint32_t)(uintptr_t)(lds_void*)&ptile[wave][0];
    const uint32_t twr = tile + (uint32_t)(l16 * kTileRow + 8 * (g ^ ((l16 >> 2) & 3)));
    // the read rows are 4g .. 4g + 3, so (row >> 2) & 3 == g
    const uint32_t trd = tile + (uint32_t)((4 * g + (l16 >> 2)) * kTileRow + 8 * ((l16 & 3) ^ g));

    // the row normalisers are written by the first wave of each head (an
    // instance of its own: the writes' addresses would otherwise hold registers)
    // (lanes g = 0 and 1 of the head's first wave: row 16 g + l16, = lane)
    const bool lse_writer = LSE && pbi == 0 && g < 2;

    int b = a.users.find_wave(v_lo);
    for (; b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int64_t nrows = s_hi - s_lo;
        const int ntiles = (int)((nrows + 31) / 32);
        const int nrows32 = (int)nrows;
        const unsigned char* kseg = uniform_ptr(Kg + gbase * krow + (int64_t)h0 * DH * 2);
        const unsigned char* vseg = uniform_ptr(Vg + gbase * vrow + (int64_t)h0 * DH * 2);

        // the flag words start clear (every wave has passed the previous
        // segment's final barrier, so none still reads them)
        if (wave == 0 && lane < 4) xflag[lane] = 0u;
        wait_lgkm0();

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
                // lane -> row (lane % 32) clamped to the segment; the aligned
                // 4-byte word holding the row's mask byte
                const uintptr_t m0 = (uintptr_t)(a.mask + gbase + r0);
                const int rr = min(lane & 31, last);
                dma4c((const void*)(m0 & ~(uintptr_t)3), (uint32_t)((int)(m0 & 3) + rr) & ~3u,
                      __builtin_amdgcn_readfirstlane(mk_lds + (uint32_t)(slot * 256)));
            }
        };
        auto unit_valid = [&](int t, int slot) -> uint32_t {
            const int64_t r0 = (int64_t)t * 32;
            const int rows_here = (int)min((int64_t)32, nrows - r0);
            bool v = lane < rows_here;
            if constexpr (MASKED) {
                const uint32_t m0 = (uint32_t)((uintptr_t)(a.mask + gbase + r0) & 3);
                const int sh = 8 * (int)((m0 + (uint32_t)min(lane & 31, rows_here - 1)) & 3);
                const uint32_t wd = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                    mk_lds + (uint32_t)(slot * 256 + 4 * lane));
                v = v && ((wd >> sh) & 0xffu) != 0;
            }
            return (uint32_t)__ballot(v);
        };

        f32x4 acc[NSB][DB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // S = P K^T of the stage in `slot`: s[half][sb][r] is the score of
        // prototype 32 pbi + 16 sb + 4 g + r and row 16 half + l16
        auto scores = [&](uint32_t sbase, f32x4 (&s)[2][NSB]) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                lds_bf16x8* p0 = klane[kc] + sbase / 16;
                const bf16x8 k0 = p0[0];
                const bf16x8 k1 = p0[16 * ROWB / 16];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    s[0][sb] = mfma(pf[sb][kc], k0, kc == 0 ? z : s[0][sb]);
                    s[1][sb] = mfma(pf[sb][kc], k1, kc == 0 ? z : s[1][sb]);
                }
            }
        };

        // The stage loop is software-pipelined: step t (after the step's one
        // block barrier) finishes stage t -- the row sums its waves published
        // in the previous step, the normalised weights, the aggregation --
        // and starts stage t + 1 -- scores, exponentials, partial row sums
        // into the other exchange buffer.  One barrier per step then orders
        // both the ring and the exchange; the ring runs two stages ahead.
        float e[2][NSB][4];       // a started stage's weights 2^(s c), front() -> back()
        uint32_t valid_c = 0;     // and its validity bits

        // start stage t (ring slot `slot`): scores, weights before
        // normalisation, this wave's partial row sums and its exact-path flag
        auto front = [&](int t, int slot) {
            const uint32_t valid = unit_valid(t, slot);
            valid_c = valid;
            // the row whose total this lane holds after rows_sum
            const int rr = l16 + 16 * (g & 1);
            const bool vr = (valid >> rr) & 1u;
            f32x4 s[2][NSB];
            scores((uint32_t)(slot * 2 * STAGE), s);
            float z[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                z[h] = 0.f;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        e[h][sb][r] = __builtin_amdgcn_exp2f(PRESCALE ? s[h][sb][r] : s[h][sb][r] * cs);
                        z[h] += e[h][sb][r];
                    }
            }
            const float zr = rows_sum(z[0], z[1]);
            // false for NaN and Inf too
            const bool fits = !vr || (zr >= kFitLo && zr <= kFitHi);
            if (__ballot(!fits) != 0 && lane == 0) xflag[t & 3] = 1u;
            if (lane < 32) xsum[t & 1][hl][pbi][lane] = zr;
        };

        // finish stage t (its row sums published before this step's barrier)
        auto back = [&](int t, int slot) {
            const uint32_t sbase = (uint32_t)(slot * 2 * STAGE);
            const uint32_t valid = valid_c;
            const bool full = valid == 0xffffffffu;
            const bool v0 = (valid >> l16) & 1u, v1 = (valid >> (16 + l16)) & 1u;
            const int xb = t & 1;
            const bool exact = xflag[t & 3] != 0u;
            // stage t + 2's flag: last read (stage t - 2) before this step's
            // barrier, next set in the following step
            if (wave == 0 && lane == 0) xflag[(t + 2) & 3] = 0u;

            // rows l16 and 16 + l16: 1 / Z, and Z with the maximum it is relative to
            float rz[2], Zr[2], Mr[2] = {0.f, 0.f};
            if (__builtin_expect(!exact, 1)) {
                float Z0 = 0.f, Z1 = 0.f;
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    Z0 += xsum[xb][hl][q][l16];
                    Z1 += xsum[xb][hl][q][16 + l16];
                }
                Zr[0] = Z0;
                Zr[1] = Z1;
            } else {
                // exact path for the stage (all waves of the block): row
                // maxima first, then sums of 2^(s c - max); the stage's keys
                // are still in the ring (its slot is refilled after the next
                // step's barrier)
                f32x4 s[2][NSB];
                scores(sbase, s);
                float x[2][NSB][4], mx[2], z[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool vh = h ? v1 : v0;
                    mx[h] = -INFINITY;
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            x[h][sb][r] = vh ? s[h][sb][r] * cs : -INFINITY;
                            mx[h] = fmaxf(mx[h], x[h][sb][r]);
                        }
                }
                const float mr = rows_max(mx[0], mx[1]);
                if (lane < 32) xmax[hl][pbi][lane] = mr;
                wait_lgkm0();
                block_barrier();
                float M[2] = {-INFINITY, -INFINITY};
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    M[0] = fmaxf(M[0], xmax[hl][q][l16]);
                    M[1] = fmaxf(M[1], xmax[hl][q][16 + l16]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (M[h] == -INFINITY) M[h] = 0.f;   // a row without a valid score
                    z[h] = 0.f;
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            e[h][sb][r] = __builtin_amdgcn_exp2f(x[h][sb][r] - M[h]);
                            z[h] += e[h][sb][r];
                        }
                }
                // this buffer's fast-path sums are not read on the exact path
                const float zx = rows_sum(z[0], z[1]);
                if (lane < 32) xsum[xb][hl][pbi][lane] = zx;
                wait_lgkm0();
                block_barrier();
                float Z0 = 0.f, Z1 = 0.f;
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    Z0 += xsum[xb][hl][q][l16];
                    Z1 += xsum[xb][hl][q][16 + l16];
                }
                Zr[0] = Z0;
                Zr[1] = Z1;
                Mr[0] = M[0];
                Mr[1] = M[1];
            }
            // invalid rows get weight 0 through 1 / Z = 0: without a mask their
            // keys are copies of the segment's last row, so 2^(s c) is finite
            // there; masked rows may hold anything and are selected below
            rz[0] = v0 ? __builtin_amdgcn_rcpf(Zr[0]) : 0.f;
            rz[1] = v1 ? __builtin_amdgcn_rcpf(Zr[1]) : 0.f;
            if (lse_writer) {
                // the row normaliser of row `lane`, natural log (-inf for masked rows)
                const int rows_here = (int)min((int64_t)32, nrows - (int64_t)t * 32);
                float* lrow = uniform_ptr(lse_out + (gbase + (int64_t)t * 32) * a.H + head);
                const bool vl = g ? v1 : v0;
                const float zl = g ? Zr[1] : Zr[0], ml = g ? Mr[1] : Mr[0];
                if (lane < rows_here) lrow[lane * a.H] = vl ? (ml + __log2f(zl)) * kLn2 : -INFINITY;
            }

            // normalised bf16 weights, transposed through the wave's tile into
            // the aggregation's B operand (k-slots = rows, as V^T's)
            bf16x8 pk[NSB];
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float p[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[r] = e[h][sb][r] * rz[h];
                    if constexpr (MASKED) {
                        const bool vh = h ? v1 : v0;
#pragma unroll
                        for (int r = 0; r < 4; ++r) p[r] = vh ? p[r] : 0.f;
                    }
                    const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                    *(lds_bf16x4*)(uintptr_t)(twr + (uint32_t)(16 * h * kTileRow)) =
                        __builtin_shufflevector(q0, q1, 0, 1, 2, 3);
                }
                union {
                    i16x4 h[2];
                    bf16x8 v;
                } pt;
                pt.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)trd);
                pt.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(trd + 16 * kTileRow));
                pk[sb] = pt.v;
            }

            // V^T operands (read after the weights, so that they and the fp32
            // weights are never live together)
            i16x4 lo[DB], hi[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                lo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vlane[db] + sbase / 8);
                hi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vlane[db] + (sbase + 16 * ROWB) / 8);
            }
            if (!full) {
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

        // step t (stage t in ring slot `slot` = t % S, a literal at every
        // call): stage t + 1 has landed and stage t's row sums are published
        // once every wave passes the barrier, which also frees slot
        // (t - 1) % S (read by step t - 1) for stage t + 3
        auto step = [&](int t, int slot) {
            wait_after<1, VMS>(max(0, min(1, ntiles - 2 - t)));
            block_barrier();
            if (t + 3 < ntiles) issue(t + 3, (slot + 3) % S);
            back(t, slot);
            if (t + 1 < ntiles) front(t + 1, (slot + 1) % S);
            // every LDS access of this step has completed before the next barrier
            wait_lgkm0();
        };
        static_assert(S == 4, "the step loop is unrolled by the ring size");
        if (0 < ntiles) issue(0, 0);
        if (1 < ntiles) issue(1, 1);
        if (2 < ntiles) issue(2, 2);
        // stage 0 has landed; then start it
        wait_after<2, VMS>(min(2, ntiles - 1));
        block_barrier();
        front(0, 0);
        wait_lgkm0();
        int t = 0;
        for (; t + S <= ntiles; t += S) {
            step(t, 0);
            step(t + 1, 1);
            step(t + 2, 2);
            step(t + 3, 3);
        }
        if (t < ntiles) step(t, 0);
        if (t + 1 < ntiles) step(t + 1, 1);
        if (t + 2 < ntiles) step(t + 2, 2);

        // segment epilogue: the weighted sums at slot w + b, lane order
        {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    store16_wt((f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH, (pbi * 32) / 16 + sb, db, lane),
                               acc[sb][db]);
        }
        wait_vm<0>();
        wait_lgkm0();
        block_barrier();
    }
}

namespace {

template <int DH, int NW, int NH>
hipError_t launch_proto(const FwdArgs& a, float* lse_out, hipStream_t s) {
    dim3 grid(a.G, a.H / NH), block(NW * 64);
    const bool m = a.mask != nullptr, l = lse_out != nullptr;
    if (m && l) hipLaunchKernelGGL((sa_proto_stream_kernel<DH, NW, NH, true, true>), grid, block, 0, s, a, lse_out);
    if (m && !l) hipLaunchKernelGGL((sa_proto_stream_kernel<DH, NW, NH, true, false>), grid, block, 0, s, a, lse_out);
    if (!m && l) hipLaunchKernelGGL((sa_proto_stream_kernel<DH, NW, NH, false, true>), grid, block, 0, s, a, lse_out);
    if (!m && !l) hipLaunchKernelGGL((sa_proto_stream_kernel<DH, NW, NH, false, false>), grid, block, 0, s, a, lse_out);
    return hipGetLastError();
}

__global__ void sa_fill_lse_kernel(float* p, int64_t n, const int32_t* status) {
    const float v = offsets_rejected(status) ? __builtin_nanf("") : -INFINITY;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

bool proto_one_pass(const StreamConfig& cfg, int dh) {
    return (dh == 32 || dh == 64) && cfg.MB == 32 && cfg.NH * cfg.PB == cfg.NW;
}

hipError_t launch_proto_stream(const FwdArgs& a, float* lse_out, const StreamConfig& cfg, hipStream_t s) {
    if (a.norm != 1 || a.q_batch_stride != 0 || a.H % cfg.NH != 0 || !proto_one_pass(cfg, a.dh))
        return hipErrorInvalidValue;
    const int dh = a.dh, NW = cfg.NW, NH = cfg.NH;
#define SA_PROTO(D_, W_, N_) \
    if (dh == D_ && NW == W_ && NH == N_) return launch_proto<D_, W_, N_>(a, lse_out, s);
    SA_PROTO(64, 16, 4) SA_PROTO(64, 8, 2) SA_PROTO(64, 8, 4) SA_PROTO(32, 16, 8) SA_PROTO(32, 8, 4) SA_PROTO(32, 8, 8)
#undef SA_PROTO
    return hipErrorInvalidValue;
}

hipError_t launch_fill_lse(float* lse_out, int64_t n, const int32_t* status, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = min((n + 255) / 256, (int64_t)2048);
    hipLaunchKernelGGL(sa_fill_lse_kernel, dim3((unsigned)blocks), dim3(256), 0, s, lse_out, n, status);
    return hipGetLastError();
}

}  // namespace sa
