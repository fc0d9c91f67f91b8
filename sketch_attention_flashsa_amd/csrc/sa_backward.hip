// sa_backward.hip -- gradients of the history-axis Sketch Attention forward
// (section 3.1 of the SequenceO1 paper; the paper trains SA end to end).  Per
// user b, head h, prototype j and valid row i, with the forward's saved
// log-sum-exp lse_j:
//     A_ji  = exp(c P_j.K_i - lse_j)          (recomputed, never stored)
//     dA_ji = dS_j . V_i,   D_j = dS_j . S_j  (= sum_i A_ji dA_ji)
//     ds_ji = A_ji (dA_ji - D_j)
//     dV_i = sum_j A_ji dS_j,  dK_i = c sum_j ds_ji P_j,  dP_j = c sum_i ds_ji K_i.
//
// Three passes:
//   sa_bwd_prep_kernel   D_j, lse_j in log2 units, and dS in bf16 (MFMA operand);
//   sa_bwd_dkdv_kernel   dK and dV.  A block owns a row range and one head; P_h
//                        and dS (bf16) of the current user sit in LDS; each wave
//                        takes 32-row tiles (two 16-row halves that share every
//                        operand read from LDS) and ALL m prototypes, so the
//                        sums over j stay inside the wave.  Scores are computed as
//                        S = P K^T (prototypes in the MFMA output rows), which
//                        is the layout in which the prototype index can be the
//                        reduction index of the next two products:
//                        computed transposed, dV^T = dS^T A^T and dK^T = P^T ds^T
//                        (dS and P as A operands read with ds_read_b64_tr_b16),
//                        so a lane's results are four consecutive dh of one row
//                        and leave in 16-byte (fp32) or 8-byte (bf16) stores.
//                        K and V fragments come straight from memory (16 bytes
//                        per lane);
//   sa_bwd_dp_kernel     dP.  Waves own (head, 32-prototype block) as in the
//                        forward; scores as S^T = K P^T (rows in the output
//                        rows), so rows are the reduction index of
//                        dP^T += K^T ds^T.  32-row K/V tiles are staged in LDS;
//                        one partial per (segment, head) like the forward's,
//                        summed in fixed order by sa_bwd_dp_merge_kernel.
// Rows past a segment's end load a clamped valid row; rows that are invalid
// (past the end, masked) get weight 0 by select, and their K values are
// zeroed before the dP product, so NaN in masked rows cannot leak.
#include <stdlib.h>

#include <type_traits>

#include "sa_device.h"

namespace sa {

using namespace dev;

// ---------------------------------------------------------------- prep
__global__ __launch_bounds__(256) void sa_bwd_prep_kernel(BwdArgs a) {
    const int64_t n = (int64_t)a.users.B * a.H * a.m;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    const float* s = a.S + t * a.dh;
    const float* gs = a.dS + t * a.dh;
    float d = 0.f;
    for (int e = 0; e < a.dh; e += 4) {
        const f32x4 x = *(const f32x4*)(s + e), y = *(const f32x4*)(gs + e);
        d += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
        bf16* o = a.dSb + t * a.dh + e;
        o[0] = (bf16)y[0];
        o[1] = (bf16)y[1];
        o[2] = (bf16)y[2];
        o[3] = (bf16)y[3];
    }
    a.Dv[t] = d;
    a.L2v[t] = a.lse[t] * kLog2e;
}

// ---------------------------------------------------------------- dK, dV
// Waves per SIMD the dK/dV kernel is compiled for (blocks of four waves, one
// per SIMD): as many as its registers allow (a wave holds two 16-row halves'
// K and V fragments, their prefetch and their dK, dV sums: ~250 registers at
// dh = 64, ~160 at dh = 32), and no more than LDS allows (P and dS of one
// head take 4 m (dh + 8) bytes).
constexpr int dkdv_occupancy(int DH, int NKB) { return DH == 32 ? 3 : 2; }

template <int DH, int NKB, bool GBF16, bool MASKED>
__global__ __launch_bounds__(256, dkdv_occupancy(DH, NKB)) void sa_bwd_dkdv_kernel(BwdArgs a) {
    constexpr int M = 32 * NKB;
    constexpr int KC = DH / 32, DB = DH / 16;
    constexpr int PS = DH + 8;                       // LDS row stride (elements)
    __shared__ __attribute__((aligned(16))) bf16 p_l[M * PS];
    __shared__ __attribute__((aligned(16))) bf16 g_l[M * PS];
    __shared__ __attribute__((aligned(16))) float l2_l[M];
    __shared__ __attribute__((aligned(16))) float d_l[M];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15, kq = l16 >> 2, q = l16 & 3;
    const int w = blockIdx.x, h = blockIdx.y;
    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G1, a.R_fixed, a.R_min, 50);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);
    const uint32_t p_base = (uint32_t)(uintptr_t)(lds_void*)p_l, g_base = (uint32_t)(uintptr_t)(lds_void*)g_l;
    // transposed reads: lane (g, kq, q) points at row 4g + kq, columns 16 db + 4q..+3
    const uint32_t tr_off = (uint32_t)(((4 * g + kq) * PS + 4 * q) * 2);
    const bf16* Pg = (const bf16*)a.P;
    const bf16* Kg = (const bf16*)a.K;
    const bf16* Vg = (const bf16*)a.V;

    for (int b = a.users.find(v_lo); b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        __syncthreads();                             // the previous segment's LDS reads are done
        const bf16* Pb = Pg + (int64_t)b * a.q_batch_stride + (int64_t)h * M * DH;
        const bf16* Gb = a.dSb + ((int64_t)b * a.H + h) * M * DH;
        for (int idx = threadIdx.x; idx < M * DH / 8; idx += 256) {
            const int r = idx / (DH / 8), c8 = idx - r * (DH / 8);
            *(bf16x8*)&p_l[r * PS + c8 * 8] = *(const bf16x8*)(Pb + r * DH + c8 * 8);
            *(bf16x8*)&g_l[r * PS + c8 * 8] = *(const bf16x8*)(Gb + r * DH + c8 * 8);
        }
        for (int j = threadIdx.x; j < M; j += 256) {
            l2_l[j] = a.L2v[((int64_t)b * a.H + h) * M + j];
            d_l[j] = a.Dv[((int64_t)b * a.H + h) * M + j];
        }
        __syncthreads();

        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int n = (int)(s_hi - s_lo);
        // K and V fragments of a 32-row tile, two 16-row halves u: B operands
        // (column = row 16 u + l16 of the tile, k = dh), and the rows' mask
        // bytes; the next tile's are loaded while this one computes.  Both
        // halves share every P and dS operand read from LDS.  Lanes past the
        // segment end take row n - 1 whole (its values and its mask byte), so
        // they compute exactly that row's gradients and their stores rewrite
        // its bytes with the same values: every lane stores, and the number
        // of memory operations per tile is fixed.
        bf16x8 kf[2][KC], vf[2][KC];
        int mf[2] = {1, 1};
        auto load_tile = [&](int t0, bf16x8 (&kk)[2][KC], bf16x8 (&vv)[2][KC], int (&mm)[2]) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t row = gbase + min(t0 + 16 * u + l16, n - 1);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    kk[u][kc] = *(const bf16x8*)(Kg + row * a.k_stride + (int64_t)h * DH + 32 * kc + 8 * g);
                    vv[u][kc] = *(const bf16x8*)(Vg + row * a.v_stride + (int64_t)h * DH + 32 * kc + 8 * g);
                }
                if (a.mask != nullptr) mm[u] = a.mask[row];
            }
        };
        if (32 * wave < n) load_tile(32 * wave, kf, vf, mf);
        // settle the first tile here: otherwise the compiler treats kf and vf
        // as loads in flight at the loop head and waits inside every tile's
        // prototype loop, which also drains the next tile's prefetch
        wait_vm<0>();
        for (int t0 = 32 * wave; t0 < n; t0 += 128) {
            bool valid[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) valid[u] = mf[u] != 0;
            bf16x8 kn[2][KC], vn[2][KC];
            int mn[2] = {1, 1};
            const bool more = t0 + 128 < n;
            if (more) load_tile(t0 + 128, kn, vn, mn);
            f32x4 dva[2][DB], dka[2][DB];
            // one block of 32 prototypes: weights and score gradients packed
            // as the B operands (column = this lane's row, k = the 32
            // prototypes in the tok_of order) of dV^T += dS^T A^T and
            // dK^T += P^T ds^T; the first block starts the sums (C = 0), so
            // they need no clearing
            auto step = [&](int kb, auto first) {
                float av[2][8], dv[2][8];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int pb = 2 * kb + half;
                    f32x4 s[2], da[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) s[u] = da[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const bf16x8 pa = *(const bf16x8*)&p_l[(16 * pb + l16) * PS + 32 * kc + 8 * g];
                        const bf16x8 ga = *(const bf16x8*)&g_l[(16 * pb + l16) * PS + 32 * kc + 8 * g];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            s[u] = mfma(pa, kf[u][kc], s[u]);
                            da[u] = mfma(ga, vf[u][kc], da[u]);
                        }
                    }
                    const f32x4 l2 = *(const f32x4*)&l2_l[16 * pb + 4 * g];
                    const f32x4 dd = *(const f32x4*)&d_l[16 * pb + 4 * g];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = __builtin_amdgcn_exp2f(fmaf(s[u][i], a.c2, -l2[i]));
                            const float y = x * (da[u][i] - dd[i]);
                            // masked rows: weight 0 by select (their values may be NaN)
                            av[u][4 * half + i] = MASKED ? (valid[u] ? x : 0.f) : x;
                            dv[u][4 * half + i] = MASKED ? (valid[u] ? y : 0.f) : y;
                        }
                }
                bf16x8 apk[2], dpk[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    apk[u] = cat8(pack2(av[u][0], av[u][1]), pack2(av[u][2], av[u][3]), pack2(av[u][4], av[u][5]),
                                  pack2(av[u][6], av[u][7]));
                    dpk[u] = cat8(pack2(dv[u][0], dv[u][1]), pack2(dv[u][2], dv[u][3]), pack2(dv[u][4], dv[u][5]),
                                  pack2(dv[u][6], dv[u][7]));
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint32_t o = tr_off + (uint32_t)((32 * kb * PS + 16 * db) * 2);
                    union {
                        i16x4 h[2];
                        bf16x8 v;
                    } gt, pt;
                    gt.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(g_base + o));
                    gt.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(g_base + o + 16 * PS * 2));
                    pt.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(p_base + o));
                    pt.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(p_base + o + 16 * PS * 2));
                    // transposed products: the lane's four results are four
                    // consecutive dh of one row
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                        dva[u][db] = mfma(gt.v, apk[u], decltype(first)::value ? zero : dva[u][db]);
                        dka[u][db] = mfma(pt.v, dpk[u], decltype(first)::value ? zero : dka[u][db]);
                    }
                }
            };
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < DB; ++db) dva[u][db] = dka[u][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int kb = 0; kb < NKB; ++kb) step(kb, std::false_type{});
            // row t0 + 16 u + l16, columns 16 db + 4 g + 0..3: one 16-byte
            // (fp32) or 8-byte (bf16) store per tensor and dh block
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t r = gbase + min(t0 + 16 * u + l16, n - 1);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int64_t o = (r * a.H + h) * DH + 16 * db + 4 * g;
                    const f32x4 dk = dka[u][db] * a.c;
                    if constexpr (GBF16) {
                        *(bf16x4*)((bf16*)a.dV + o) = __builtin_convertvector(dva[u][db], bf16x4);
                        *(bf16x4*)((bf16*)a.dK + o) = __builtin_convertvector(dk, bf16x4);
                    } else {
                        *(f32x4*)((float*)a.dV + o) = dva[u][db];
                        *(f32x4*)((float*)a.dK + o) = dk;
                    }
                }
            }
            if (more) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        kf[u][kc] = kn[u][kc];
                        vf[u][kc] = vn[u][kc];
                    }
                    mf[u] = mn[u];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- dP
template <int DH>
__global__ __launch_bounds__(512) void sa_bwd_dp_kernel(BwdArgs a, int NH, int PB) {
    constexpr int KC = DH / 32, DB = DH / 16, NSB = 2;
    constexpr int TS = kBwdTileCols + 8;            // LDS row stride of the K/V tile (elements)
    __shared__ __attribute__((aligned(16))) bf16 kt[2][32 * TS];   // double-buffered tiles
    __shared__ __attribute__((aligned(16))) bf16 vt[2][32 * TS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15, kq = l16 >> 2, q = l16 & 3;
    const int nthreads = NH * PB * 64;
    const int w = blockIdx.x;
    const int h0 = blockIdx.y * NH;
    const int hl = wave / PB, pb = wave - hl * PB;
    const int head = h0 + hl;
    const bool active = head < a.H;
    const int cols = NH * DH;                        // tile columns actually used

    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, 50);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);
    const bf16* Pg = (const bf16*)a.P;
    const bf16* Kg = (const bf16*)a.K;
    const bf16* Vg = (const bf16*)a.V;
    const uint32_t k_base = (uint32_t)(uintptr_t)(lds_void*)&kt[0][0];
    const uint32_t tr_off = (uint32_t)(((4 * g + kq) * TS + hl * DH + 4 * q) * 2);

    for (int b = a.users.find(v_lo); b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int n = (int)(s_hi - s_lo);
        const int hh = active ? head : h0;
        // B operands: column = prototype 32 pb + 16 sb + l16, k = dh
        bf16x8 pf[NSB][KC], gf[NSB][KC];
        float l2v[NSB], dv[NSB];
        const bf16* Pb = Pg + (int64_t)b * a.q_batch_stride + (int64_t)hh * a.m * DH;
        const bf16* Gb = a.dSb + ((int64_t)b * a.H + hh) * a.m * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int j = 32 * pb + 16 * sb + l16;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                pf[sb][kc] = *(const bf16x8*)(Pb + (int64_t)j * DH + 32 * kc + 8 * g);
                gf[sb][kc] = *(const bf16x8*)(Gb + (int64_t)j * DH + 32 * kc + 8 * g);
            }
            l2v[sb] = a.L2v[((int64_t)b * a.H + hh) * a.m + j];
            dv[sb] = a.Dv[((int64_t)b * a.H + hh) * a.m + j];
        }
        f32x4 acc[NSB][DB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // the block stages 32-row K/V tiles in LDS; tile t + 1 is loaded into
        // registers while tile t is computed, and written after a barrier
        // 16-byte chunks per tile per tensor: 4 NH dh of them for NH PB waves,
        // so at most dh / (16 PB) <= 4 per thread
        const int nchunk = 32 * cols / 8;
        const int per = (nchunk + nthreads - 1) / nthreads;
        bf16x8 kreg[4], vreg[4];
        auto load_tile = [&](int t0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int idx = threadIdx.x + u * nthreads;
                if (u < per && idx < nchunk) {
                    const int r = idx / (cols / 8), c8 = idx - r * (cols / 8);
                    const int64_t row = gbase + min(t0 + r, n - 1);
                    kreg[u] = *(const bf16x8*)(Kg + row * a.k_stride + (int64_t)h0 * DH + c8 * 8);
                    vreg[u] = *(const bf16x8*)(Vg + row * a.v_stride + (int64_t)h0 * DH + c8 * 8);
                }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int idx = threadIdx.x + u * nthreads;
                if (u < per && idx < nchunk) {
                    const int r = idx / (cols / 8), c8 = idx - r * (cols / 8);
                    *(bf16x8*)&kt[buf][r * TS + c8 * 8] = kreg[u];
                    *(bf16x8*)&vt[buf][r * TS + c8 * 8] = vreg[u];
                }
            }
        };
        // tile t lives in buffer t & 1; tile t + 1 is loaded into registers
        // while tile t is computed and stored into the other buffer (read by
        // tile t - 1, done before the previous barrier): one barrier per tile
        load_tile(0);
        store_tile(0);
        __syncthreads();
        for (int t0 = 0, it = 0; t0 < n; t0 += 32, ++it) {
            const int cur = it & 1;
            const bool more = t0 + 32 < n;
            if (more) load_tile(t0 + 32);
            if (active) {
                // validity of the tile's 32 rows (bit r)
                const int tl = t0 + lane;
                bool vr = lane < 32 && tl < n;
                if (a.mask) vr = vr && a.mask[gbase + min(tl, n - 1)] != 0;
                const uint32_t valid = (uint32_t)__ballot(vr);
                // S^T = K P^T and dA^T = V dS^T: rows = tokens (two 16-row halves)
                f32x4 s[2][NSB], da[2][NSB];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) s[half][sb] = da[half][sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const bf16x8 kr = *(const bf16x8*)&kt[cur][(16 * half + l16) * TS + hl * DH + 32 * kc + 8 * g];
                        const bf16x8 vr8 = *(const bf16x8*)&vt[cur][(16 * half + l16) * TS + hl * DH + 32 * kc + 8 * g];
#pragma unroll
                        for (int sb = 0; sb < NSB; ++sb) {
                            s[half][sb] = mfma(kr, pf[sb][kc], s[half][sb]);
                            da[half][sb] = mfma(vr8, gf[sb][kc], da[half][sb]);
                        }
                    }
                }
                // ds^T packed as the B operand of dP^T += K^T ds^T (k = tokens in the
                // tok_of order, column = prototype)
                const uint32_t vj = lane_slots(valid, g);
                bf16x8 pk[NSB];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    float x[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const float sc = s[jj >> 2][sb][jj & 3], dd = da[jj >> 2][sb][jj & 3];
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc, a.c2, -l2v[sb]));
                        x[jj] = ((vj >> jj) & 1) ? p * (dd - dv[sb]) : 0.f;
                    }
                    pk[sb] = cat8(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    union {
                        i16x4 h[2];
                        bf16x8 v;
                    } kT;
                    const uint32_t o = k_base + (uint32_t)(cur * 32 * TS * 2) + tr_off + (uint32_t)(16 * db * 2);
                    kT.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)o);
                    kT.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(o + 16 * TS * 2));
                    if (valid != 0xffffffffu) {
                        // invalid rows: zero their keys (NaN in masked rows must not leak)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            if (!((vj >> jj) & 1)) kT.h[0][jj] = 0;
                            if (!((vj >> (4 + jj)) & 1)) kT.h[1][jj] = 0;
                        }
                    }
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) acc[sb][db] = mfma(kT.v, pk[sb], acc[sb][db]);
                }
            }
            if (more) store_tile(cur ^ 1);
            __syncthreads();
        }
        if (active) {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *(f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH, 2 * pb + sb, db, lane) =
                        acc[sb][db] * a.c;
        }
    }
}

// The same dP computation fed by a direct-to-LDS ring (the forward streaming
// kernel's scheme): K and V rows of the block's heads (CPR 16-byte chunks per
// row per tensor) stream through kDpStages 32-row stages, kDpStages - 1 of
// them in flight while one is computed, each wave waiting (counted vmcnt)
// for its own loads before the block barrier.  K is read row-wise for the
// scores and transposed for dP^T += K^T ds^T, V row-wise for dA, so both
// tensors take one XOR swizzle of the 16-byte chunks, dp_swz(row % 16), under
// which a 16-lane group of row reads touches 16 distinct chunks of the
// 256-byte bank window and a 32-lane group of transposed reads 8 distinct
// 32-byte chunk pairs.  Compiled for 8-wave blocks (NH heads x PB prototype
// blocks = 8) with NH dh = 8 CPR in {128, 256}.
namespace {
constexpr int kDpStages = 4;
__device__ __forceinline__ int dp_swz(int r) { return 2 * (r & 7) + ((r >> 3) & 1); }
}  // namespace

template <int DH, int CPR, bool MASKED>
__global__ __launch_bounds__(512, CPR == 16 ? 2 : 1) void sa_bwd_dp_stream_kernel(BwdArgs a, int NH, int PB) {
    constexpr int KC = DH / 32, DB = DH / 16, NSB = 2, NW = 8;
    constexpr int S = kDpStages, AHEAD = S - 1;
    constexpr int ROWB = CPR * 16;                   // bytes per row per tensor
    constexpr int STAGE = 32 * ROWB;                 // bytes per tensor per stage
    constexpr int D = 32 * CPR / (NW * 64);          // DMA ops per wave per tensor per stage
    // K and V, and with a mask one 4-byte load of the stage's mask words
    constexpr int VMS = 2 * D + (MASKED ? 1 : 0);
    static_assert(D >= 1 && D * NW * 64 == 32 * CPR, "a stage is whole DMA ops per wave");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[S][2][STAGE];
    // with a mask: each wave's own copy of a stage's mask words, lane i < 32
    // holding the aligned 4-byte word that contains row i's byte (a plain
    // load at the point of use would make the compiler, which cannot count
    // the ring's asm loads, drain the ring)
    __shared__ __attribute__((aligned(16))) uint32_t mkring[MASKED ? S : 1][MASKED ? NW * 64 : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15, kq = l16 >> 2, q = l16 & 3;
    const int w = blockIdx.x;
    const int h0 = blockIdx.y * NH;
    const int hl = wave / PB, pb = wave - hl * PB;
    const int head = h0 + hl;
    const bool active = head < a.H;

    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, 50);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);
    const bf16* Pg = (const bf16*)a.P;
    const unsigned char* Kg = (const unsigned char*)a.K;
    const unsigned char* Vg = (const unsigned char*)a.V;
    const int64_t krow = a.k_stride * 2, vrow = a.v_stride * 2;

    // per-lane DMA geometry: op (wave D + d) writes 1 KB of the stage; lane
    // writes 16 B at row * ROWB + slot * 16 and fetches the logical chunk the
    // swizzle places there
    int dma_row[D], dma_ck[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int off = (wave * D + d) * 1024 + lane * 16;
        dma_row[d] = off / ROWB;
        dma_ck[d] = (((off % ROWB) / 16) ^ dp_swz(dma_row[d] & 15)) * 16;
    }
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0][0];
    const uint32_t mk_lds = (uint32_t)(uintptr_t)(lds_void*)&mkring[0][0];
    const int hc = min(h0 + hl, a.H - 1) - h0;      // head column of this wave (clamped for idle waves)
    uint32_t rd[KC];                                 // row reads: row l16, chunk hc dh/8 + 4 kc + g
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
        rd[kc] = (uint32_t)(l16 * ROWB + (((hc * (DH / 8) + 4 * kc + g) ^ dp_swz(l16)) * 16));
    uint32_t tr[DB];                                 // transposed reads: row 4 g + kq, channels 16 db + 4 q
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int row = 4 * g + kq, c = hc * (DH / 8) + 2 * db + (q >> 1);
        tr[db] = (uint32_t)(row * ROWB + ((c ^ dp_swz(row)) * 16) + 8 * (q & 1));
    }

    for (int b = a.users.find(v_lo); b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int n = (int)(s_hi - s_lo);
        const int ntiles = (n + 31) / 32;
        const int hh = active ? head : h0;
        // B operands: column = prototype 32 pb + 16 sb + l16, k = dh
        bf16x8 pf[NSB][KC], gf[NSB][KC];
        float l2v[NSB], dv[NSB];
        const bf16* Pb = Pg + (int64_t)b * a.q_batch_stride + (int64_t)hh * a.m * DH;
        const bf16* Gb = a.dSb + ((int64_t)b * a.H + hh) * a.m * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int j = 32 * pb + 16 * sb + l16;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                pf[sb][kc] = *(const bf16x8*)(Pb + (int64_t)j * DH + 32 * kc + 8 * g);
                gf[sb][kc] = *(const bf16x8*)(Gb + (int64_t)j * DH + 32 * kc + 8 * g);
            }
            l2v[sb] = a.L2v[((int64_t)b * a.H + hh) * a.m + j];
            dv[sb] = a.Dv[((int64_t)b * a.H + hh) * a.m + j];
        }
        // settle these loads before the ring's counted waits start
        wait_vm<0>();
        f32x4 acc[NSB][DB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};

        const unsigned char* kseg = Kg + gbase * krow + (int64_t)h0 * DH * 2;
        const unsigned char* vseg = Vg + gbase * vrow + (int64_t)h0 * DH * 2;
        auto issue = [&](int t) {
            const uint32_t slot = ring_lds + (uint32_t)((t % S) * 2 * STAGE) + (uint32_t)(wave * D * 1024);
            const int last = n - 1 - t * 32;         // rows past the segment end re-read its last row
            const unsigned char* kb = kseg + (int64_t)t * 32 * krow;
            const unsigned char* vb = vseg + (int64_t)t * 32 * vrow;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int rr = min(dma_row[d], last);
                dma16c(kb, (uint32_t)(rr * (int)krow + dma_ck[d]), __builtin_amdgcn_readfirstlane(slot + d * 1024));
                dma16c(vb, (uint32_t)(rr * (int)vrow + dma_ck[d]),
                       __builtin_amdgcn_readfirstlane(slot + STAGE + d * 1024));
            }
            if constexpr (MASKED) {
                // lane -> row (lane % 32) clamped to the segment: the aligned
                // word around its mask byte (never leaves the byte's page)
                const uintptr_t m0 = (uintptr_t)(a.mask + gbase + (int64_t)t * 32);
                const int rr = min(lane & 31, last);
                dma4c((const void*)(m0 & ~(uintptr_t)3), (uint32_t)((int)(m0 & 3) + rr) & ~3u,
                      __builtin_amdgcn_readfirstlane(mk_lds + (uint32_t)(((t % S) * NW + wave) * 256)));
            }
        };

#pragma unroll
        for (int t = 0; t < AHEAD; ++t)
            if (t < ntiles) issue(t);
        for (int t = 0; t < ntiles; ++t) {
            // this wave's part of stage t has landed; the barrier makes the
            // stage complete and frees slot (t - 1) % S for stage t + AHEAD
            wait_after<AHEAD - 1, VMS>(min(AHEAD - 1, ntiles - 1 - t));
            block_barrier();
            if (t + AHEAD < ntiles) issue(t + AHEAD);
            if (active) {
                const uint32_t kst = ring_lds + (uint32_t)((t % S) * 2 * STAGE), vst = kst + STAGE;
                const int tl = t * 32 + lane;
                bool vr = lane < 32 && tl < n;
                if constexpr (MASKED) {
                    const uint32_t m0 = (uint32_t)((uintptr_t)(a.mask + gbase + (int64_t)t * 32) & 3);
                    const int sh = 8 * (int)((m0 + (uint32_t)min(lane & 31, n - 1 - t * 32)) & 3);
                    const uint32_t wd = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                        mk_lds + (uint32_t)(((t % S) * NW + wave) * 256 + 4 * lane));
                    vr = vr && ((wd >> sh) & 0xffu) != 0;
                }
                const uint32_t valid = (uint32_t)__ballot(vr);
                // S^T = K P^T and dA^T = V dS^T: rows = tokens (two 16-row halves)
                f32x4 s[2][NSB], da[2][NSB];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) s[half][sb] = da[half][sb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const uint32_t o = rd[kc] + (uint32_t)(16 * half * ROWB);
                        const bf16x8 kr = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(kst + o);
                        const bf16x8 vr8 = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(vst + o);
#pragma unroll
                        for (int sb = 0; sb < NSB; ++sb) {
                            s[half][sb] = mfma(kr, pf[sb][kc], s[half][sb]);
                            da[half][sb] = mfma(vr8, gf[sb][kc], da[half][sb]);
                        }
                    }
                }
                // ds^T packed as the B operand of dP^T += K^T ds^T (k = tokens in
                // the tok_of order, column = prototype)
                const uint32_t vj = lane_slots(valid, g);
                bf16x8 pk[NSB];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    float x[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const float sc = s[jj >> 2][sb][jj & 3], dd = da[jj >> 2][sb][jj & 3];
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc, a.c2, -l2v[sb]));
                        x[jj] = ((vj >> jj) & 1) ? p * (dd - dv[sb]) : 0.f;
                    }
                    pk[sb] = cat8(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    union {
                        i16x4 h[2];
                        bf16x8 v;
                    } kT;
                    kT.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(kst + tr[db]));
                    kT.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(uintptr_t)(kst + tr[db] + 16 * ROWB));
                    if (valid != 0xffffffffu) {
                        // invalid rows: zero their keys (NaN in masked rows must not leak)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            if (!((vj >> jj) & 1)) kT.h[0][jj] = 0;
                            if (!((vj >> (4 + jj)) & 1)) kT.h[1][jj] = 0;
                        }
                    }
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) acc[sb][db] = mfma(kT.v, pk[sb], acc[sb][db]);
                }
            }
            // every LDS read of this stage has completed before the next barrier
            wait_lgkm0();
        }
        if (active) {
            const int64_t slot = (int64_t)w + b;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *(f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH, 2 * pb + sb, db, lane) =
                        acc[sb][db] * a.c;
        }
        // drain this segment's loads and let every wave finish reading the
        // ring before the next segment's prologue refills it
        wait_vm<0>();
        wait_lgkm0();
        block_barrier();
    }
}

// dP = sum of the dP partials of the segments in fixed order: per user (per-user
// prototypes) or over all users (shared prototypes).  One thread per four
// outputs (h, j, e..e+3); the partials are lane-major.
__global__ __launch_bounds__(256) void sa_bwd_dp_merge_kernel(BwdArgs a) {
    const int h = blockIdx.y, bo = blockIdx.z;        // bo: user (per-user P) or 0
    const int qd = blockIdx.x * 256 + threadIdx.x;
    if (qd >= a.m * (a.dh / 4)) return;
    const int lane = qd & 63, blk = qd >> 6;
    const int db = blk % (a.dh / 16), j16 = blk / (a.dh / 16);
    const int j = 16 * j16 + (lane & 15), e = 16 * db + 4 * (lane >> 4);
    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, 50);
    const int64_t md = (int64_t)a.m * a.dh;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int b0 = a.per_user ? bo : 0, b1 = a.per_user ? bo + 1 : a.users.B;
    for (int b = b0; b < b1; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (ue <= us) continue;
        const int64_t w0 = rs.range_of(us), w1 = rs.range_of(ue - 1);
        // eight segments per batch, their loads issued together (slots past
        // the last re-read it and are masked), added in ascending order
        const float* base = a.part.acc + ((int64_t)b * a.H + h) * md + (int64_t)qd * 4;
        const int64_t hmd = (int64_t)a.H * md;
        for (int64_t x0 = w0; x0 <= w1; x0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = *(const f32x4*)(base + min(x0 + k, w1) * hmd);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (x0 + k <= w1) acc += v[k];
        }
    }
    float* o = a.dP + (((int64_t)bo * a.H + h) * a.m + j) * a.dh + e;
    *(f32x4*)o = acc;
}

bool bwd_supported(int dh, int m) { return (dh == 32 || dh == 64) && (m == 32 || m == 64 || m == 128 || m == 256); }

// waves per head in the dP kernel (one per 32 prototypes) and heads per block
void bwd_dp_shape(int m, int H, int* NH, int* PB) {
    *PB = m / 32;
    int nh = 8 / *PB;
    if (nh < 1) nh = 1;
    while (nh > 1 && (H % nh != 0 || nh * 64 > kBwdTileCols)) nh >>= 1;
    *NH = nh;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
    if (a.users.B == 0) return hipSuccess;
    const int64_t n = (int64_t)a.users.B * a.H * a.m;
    hipLaunchKernelGGL(sa_bwd_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    const dim3 g1(a.G1, a.H);
    const bool masked = a.mask != nullptr;
#define SA_DKDV(D_, K_)                                                                                          \
    if (a.dh == D_ && a.m == 32 * K_) {                                                                          \
        if (a.grads_bf16 && masked) hipLaunchKernelGGL((sa_bwd_dkdv_kernel<D_, K_, true, true>), g1, dim3(256), 0, s, a); \
        if (a.grads_bf16 && !masked) hipLaunchKernelGGL((sa_bwd_dkdv_kernel<D_, K_, true, false>), g1, dim3(256), 0, s, a); \
        if (!a.grads_bf16 && masked) hipLaunchKernelGGL((sa_bwd_dkdv_kernel<D_, K_, false, true>), g1, dim3(256), 0, s, a); \
        if (!a.grads_bf16 && !masked) hipLaunchKernelGGL((sa_bwd_dkdv_kernel<D_, K_, false, false>), g1, dim3(256), 0, s, a); \
    }
    SA_DKDV(32, 1) SA_DKDV(32, 2) SA_DKDV(32, 4) SA_DKDV(32, 8) SA_DKDV(64, 1) SA_DKDV(64, 2) SA_DKDV(64, 4)
    SA_DKDV(64, 8)
#undef SA_DKDV
    int NH, PB;
    bwd_dp_shape(a.m, a.H, &NH, &PB);
    const dim3 g2(a.G, (a.H + NH - 1) / NH), blk2(NH * PB * 64);
    // the ring-fed kernel for 8-wave blocks whose rows are 128 or 256 elements
    // (K and V row starts 16-byte aligned), the register-staged one otherwise
    const int cpr = NH * a.dh / 8;
    const bool ring_ok = NH * PB == 8 && (cpr == 16 || cpr == 32) && a.k_stride % 8 == 0 && a.v_stride % 8 == 0 &&
                         !a.dp_register_staged;
#define SA_DP_RING(D_, C_)                                                                                   \
    if (masked) hipLaunchKernelGGL((sa_bwd_dp_stream_kernel<D_, C_, true>), g2, blk2, 0, s, a, NH, PB);      \
    else hipLaunchKernelGGL((sa_bwd_dp_stream_kernel<D_, C_, false>), g2, blk2, 0, s, a, NH, PB);
    if (ring_ok && a.dh == 32 && cpr == 16) { SA_DP_RING(32, 16) }
    else if (ring_ok && a.dh == 32 && cpr == 32) { SA_DP_RING(32, 32) }
    else if (ring_ok && a.dh == 64 && cpr == 16) { SA_DP_RING(64, 16) }
    else if (ring_ok && a.dh == 64 && cpr == 32) { SA_DP_RING(64, 32) }
#undef SA_DP_RING
    else if (a.dh == 32) hipLaunchKernelGGL(sa_bwd_dp_kernel<32>, g2, blk2, 0, s, a, NH, PB);
    else hipLaunchKernelGGL(sa_bwd_dp_kernel<64>, g2, blk2, 0, s, a, NH, PB);
    const int mq = a.m * (a.dh / 4);
    hipLaunchKernelGGL(sa_bwd_dp_merge_kernel, dim3((mq + 255) / 256, a.H, a.per_user ? a.users.B : 1), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace sa
