// sa_bf16_fwd.hip -- streaming Sketch Attention forward for bf16 inputs on
// gfx950 (MI355X), the FlashSA computation of section 4.4 of the SequenceO1
// paper: score blocks, running softmax statistics and aggregation fused, the
// m x n score matrix kept in registers.
//
// Block = one row range w (see sa_internal.h) x one group of NW
// (head, 16*NSB-prototype block) units, one unit per wave.  Per 32-row tile:
//   1. all threads stage the tile's K and V rows of the block's heads in LDS
//      (16-byte coalesced loads; the next tile's loads are in flight while the
//      current one is computed; rows outside the segment or masked are zeros);
//   2. each wave computes S^T[32 rows x MB prototypes] = K P^T with
//      v_mfma_f32_16x16x32_bf16 (its P fragments live in registers);
//   3. softmax over the history axis, online: p = 2^(s*c - M) with c =
//      scale*log2(e).  M only moves when a tile would exceed 2^16 (the
//      check is on each lane's partial sum of the tile), so the common path is
//      one FMA, one v_exp_f32, half a v_cvt_pk_bf16_f32 and half a
//      v_dot2c_f32_bf16 (the running sum) per score;
//   4. O^T[dh x MB] += V^T p^T with the same MFMA, p in bf16, fp32 accumulate.
// In MFMA terms each lane owns one prototype column of S^T and O^T, so the
// running statistics and the rescale factor are lane-local.
// Prototype-axis mode reuses the same loop with a per-row normaliser
// computed beforehand (sa_tok_lse.hip) and no running statistics.
#include <stdio.h>
#include <stdlib.h>

#include "sa_internal.h"

namespace sa {

namespace {

// Fast path while every weight of a tile stays <= 2^16 relative to the
// running maximum; a larger tile sum triggers the exact rescaling path.
constexpr float kLazyBound = 65536.0f;

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 pack2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ bf16x8 cat8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
    bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float dot2sum(bf16x2 a, float acc) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(a, one, acc, false);
}

__device__ __forceinline__ float xor_max(float x, int mask) {
    return fmaxf(x, __shfl_xor(x, mask, 64));
}

// Token of k-slot j (0..7) of lane group g in the PV contraction: the two
// 16-row halves of S^T give a lane rows 4g..4g+3 and 16+4g..16+4g+3.
__device__ __forceinline__ int tok_of(int g, int j) { return (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4); }

}  // namespace

template <int DH, int MB, int NW, bool PROTO>
__global__ __launch_bounds__(NW * 64) void sa_bf16_fwd_kernel(FwdArgs a, int PB, int units, int kRow, int vRow) {
    constexpr int NSB = MB / 16;          // 16-prototype sub-blocks per wave
    constexpr int KC = DH / 32;           // k-chunks of the score MFMA
    constexpr int DB = DH / 16;           // 16-wide dh blocks of the value MFMA
    constexpr int NT = NW * 64;
    constexpr int LPT = (DH / 16 + 0);    // max 16-byte loads per thread per tensor (heads <= NW)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    if (offsets_rejected(a.status)) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;              // lane group: row quad / k octet
    const int l16 = lane & 15;
    const int w = blockIdx.x;
    const int group = blockIdx.y;

    // ---- block geometry
    const int u0 = group * NW;
    const int h0 = u0 / PB;
    const int hlast = min((u0 + NW - 1) / PB, a.H - 1);
    const int NHB = hlast - h0 + 1;
    const int cpr = NHB * DH / 8;         // 16-byte chunks per row per tensor
    const int chunks = kTile * cpr;

    const int u = u0 + wave;
    const bool active = u < units;
    const int head = active ? u / PB : h0;
    const int pb = active ? u % PB : 0;
    const int hl = head - h0;

    unsigned char* Ks = smem;                              // [2][32][kRow]
    unsigned char* Vs = smem + 2 * kTile * kRow;           // [2][32][vRow]

    // ---- row range of this block
    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, a.split);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);

    const bf16* Pg = (const bf16*)a.P;
    const bf16* Kg = (const bf16*)a.K;
    const bf16* Vg = (const bf16*)a.V;

    // prototype fragments (B operand of S^T = K P^T): lane holds P[j][32kc + 8g .. +8]
    bf16x8 pf[NSB][KC];
    auto load_p = [&](int b) {
        const bf16* base = Pg + (int64_t)b * a.q_batch_stride + ((int64_t)head * a.m + pb * MB) * DH;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                pf[sb][kc] = *(const bf16x8*)(base + (int64_t)(16 * sb + l16) * DH + 32 * kc + 8 * g);
    };
    if (a.q_batch_stride == 0) load_p(0);

    u32x4 kreg[LPT], vreg[LPT];
    uint64_t valid_next = 0;
    int it = 0;  // running tile counter: LDS buffer parity across segments

    int b = a.users.find(v_lo);
    for (; b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        if (a.q_batch_stride != 0) load_p(b);
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);   // buffer row of segment row 0
        const int64_t nrows = s_hi - s_lo;
        const int ntiles = (int)((nrows + kTile - 1) / kTile);

        // running statistics (history axis) and accumulators
        float Mc[NSB], Zs[NSB];
        f32x4 acc[NSB][DB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            Mc[sb] = -INFINITY;
            Zs[sb] = 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[sb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // issue the global loads of tile t into registers; returns its validity bits
        auto prefetch = [&](int t) -> uint64_t {
            const int64_t r0 = (int64_t)t * kTile;
            const int rows_here = (int)min((int64_t)kTile, nrows - r0);
#pragma unroll
            for (int k = 0; k < LPT; ++k) {
                const int c = threadIdx.x + k * NT;
                const int r = c / cpr, col = c - r * cpr;
                bool ok = c < chunks && r < rows_here;
                const int64_t grow = gbase + r0 + r;
                if (ok && a.mask) ok = a.mask[grow] != 0;
                if (ok) {
                    const int hh = col / (DH / 8), e8 = col - hh * (DH / 8);
                    kreg[k] = *(const u32x4*)(Kg + grow * a.k_stride + (int64_t)(h0 + hh) * DH + e8 * 8);
                    vreg[k] = *(const u32x4*)(Vg + grow * a.v_stride + (int64_t)(h0 + hh) * DH + e8 * 8);
                } else {
                    kreg[k] = (u32x4){0u, 0u, 0u, 0u};
                    vreg[k] = (u32x4){0u, 0u, 0u, 0u};
                }
            }
            bool vrow = lane < rows_here;
            if (vrow && a.mask) vrow = a.mask[gbase + r0 + lane] != 0;
            return __ballot(vrow);
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int k = 0; k < LPT; ++k) {
                const int c = threadIdx.x + k * NT;
                if (c < chunks) {
                    const int r = c / cpr, col = c - r * cpr;
                    *(u32x4*)(Ks + (buf * kTile + r) * kRow + col * 16) = kreg[k];
                    // V rows are only 8-byte aligned (see vRow): two 8-byte stores
                    uint2* vd = (uint2*)(Vs + (buf * kTile + r) * vRow + col * 16);
                    vd[0] = make_uint2(vreg[k][0], vreg[k][1]);
                    vd[1] = make_uint2(vreg[k][2], vreg[k][3]);
                }
            }
        };

        valid_next = prefetch(0);
        for (int t = 0; t < ntiles; ++t, ++it) {
            const int buf = it & 1;
            const uint64_t valid = valid_next;
            store(buf);
            __syncthreads();
            if (t + 1 < ntiles) valid_next = prefetch(t + 1);
            if (!active) continue;

            const unsigned char* Kt = Ks + buf * kTile * kRow + hl * DH * 2;
            const unsigned char* Vt = Vs + buf * kTile * vRow + hl * DH * 2;

            // ---- S^T = K P^T : s[st][sb] holds rows 16st + 4g + i, prototype l16 of sub-block sb
            f32x4 s[2][NSB];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 ka[KC];
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
                    ka[kc] = *(const bf16x8*)(Kt + (16 * st + l16) * kRow + (32 * kc + 8 * g) * 2);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    f32x4 d = mfma16x16x32(ka[0], pf[sb][0], (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int kc = 1; kc < KC; ++kc) d = mfma16x16x32(ka[kc], pf[sb][kc], d);
                    s[st][sb] = d;
                }
            }

            // ---- weights p (bf16) in PV k-order: slots 0..3 rows 4g+i, slots 4..7 rows 16+4g+i
            bf16x8 pk[NSB];
            const bool full = (uint32_t)valid == 0xffffffffu;
            if constexpr (PROTO) {
                // per-row normaliser over the m prototypes (log2 units)
                float nl[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tk = tok_of(g, j);
                    const bool vd = (valid >> tk) & 1;
                    nl[j] = vd ? a.lse2_tok[(gbase + (int64_t)t * kTile + tk) * a.H + head] : 0.f;
                }
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    float p[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int tk = tok_of(g, j);
                        const float sv = s[j >> 2][sb][j & 3];
                        p[j] = ((valid >> tk) & 1) ? __builtin_amdgcn_exp2f(fmaf(sv, a.c, -nl[j])) : 0.f;
                    }
                    pk[sb] = cat8(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
                }
            } else {
                bool ok = false;
                float zt[NSB];
                if (full) {
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
                        fits = fits && (zt[sb] <= kLazyBound);   // false for NaN and Inf too
                    }
                    ok = __all(fits);
                }
                if (ok) {
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) Zs[sb] += zt[sb];
                } else {
                    // exact path: masked/partial tile, first tile, or a new maximum
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) {
                        float x[8];
                        float tm = -INFINITY;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int tk = tok_of(g, j);
                            x[j] = ((valid >> tk) & 1) ? s[j >> 2][sb][j & 3] * a.c : -INFINITY;
                            tm = fmaxf(tm, x[j]);
                        }
                        tm = xor_max(tm, 16);
                        tm = xor_max(tm, 32);
                        const float Mold = Mc[sb];
                        const float Mnew = fmaxf(Mold, tm);
                        const float f = (Mnew == Mold) ? 1.f : __builtin_amdgcn_exp2f(Mold - Mnew);
                        float p[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int tk = tok_of(g, j);
                            p[j] = ((valid >> tk) & 1) ? __builtin_amdgcn_exp2f(x[j] - Mnew) : 0.f;
                        }
                        const bf16x2 q0 = pack2(p[0], p[1]), q1 = pack2(p[2], p[3]);
                        const bf16x2 q2 = pack2(p[4], p[5]), q3 = pack2(p[6], p[7]);
                        pk[sb] = cat8(q0, q1, q2, q3);
                        Zs[sb] = Zs[sb] * f + dot2sum(q3, dot2sum(q2, dot2sum(q1, dot2sum(q0, 0.f))));
                        Mc[sb] = Mnew;
#pragma unroll
                        for (int db = 0; db < DB; ++db) acc[sb][db] *= f;
                    }
                }
            }

            // ---- O^T += V^T p^T : lane (dh 16db + l16, k-slots of group g)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const unsigned short* vcol = (const unsigned short*)(Vt + (16 * db + l16) * 2);
                union {
                    unsigned short h[8];
                    bf16x8 v;
                } vt;
#pragma unroll
                for (int j = 0; j < 8; ++j) vt.h[j] = vcol[tok_of(g, j) * (vRow / 2)];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) acc[sb][db] = mfma16x16x32(vt.v, pk[sb], acc[sb][db]);
            }
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
                for (int db = 0; db < DB; ++db)
                    __builtin_nontemporal_store(
                        acc[sb][db], (f32x4*)lane_major_acc(a.part, slot, a.H, head, a.m, DH, (pb * MB) / 16 + sb, db, lane));
            }
        }
    }
}

namespace {

void fill_config(int dh, int H, int mb, int nw, int pb, Bf16Config* cfg) {
    const int units = H * pb;
    int heads = 1;
    for (int u0 = 0; u0 < units; u0 += nw) {
        const int h0 = u0 / pb, h1 = min((u0 + nw - 1) / pb, H - 1);
        heads = max(heads, h1 - h0 + 1);
    }
    cfg->protos_per_wave = mb;
    cfg->waves = nw;
    cfg->blocks_per_cu = (nw == 8) ? 1 : 2;
    cfg->max_heads = heads;
    // LDS row strides: +16 B keeps 8 rows of 16-byte K reads on distinct banks,
    // +8 B spreads the 2-byte V^T column reads of the four lane groups
    cfg->k_row = heads * dh * 2 + 16;
    cfg->v_row = heads * dh * 2 + 8;
    cfg->lds_bytes = (size_t)2 * kTile * (cfg->k_row + cfg->v_row);
}

}  // namespace

// Tile selection.  Register budget decides it: at 8 waves per block a wave
// has 256 VGPRs, at 4 waves (one per SIMD) 512 with the accumulation
// registers; the choices below are the instantiations that do not spill.
// A requested tile (tile_mb, tile_nw) overrides the choice when valid.
bool bf16_config(int dh, int m, int H, size_t lds_limit, int tile_mb, int tile_nw, Bf16Config* cfg) {
    if (!(dh == 32 || dh == 64 || dh == 128) || m % 16 != 0) return false;
    int mb, nw;
    if (dh == 32) {
        mb = (m % 32 == 0) ? 32 : 16;
    } else {
        mb = 16;
    }
    int units = H * (m / mb);
    nw = (units % 8 == 0 && dh <= 64) ? 8 : 4;
    {
        const int emb = tile_mb, enw = tile_nw;
        if ((emb == 16 || emb == 32 || emb == 64) && m % emb == 0 && (enw == 4 || enw == 8) &&
            !(dh == 128 && (emb == 64 || enw == 8))) {
            mb = emb;
            nw = enw;
        }
    }
    const int pb = m / mb;
    fill_config(dh, H, mb, nw, pb, cfg);
    if (cfg->lds_bytes > lds_limit && nw == 8) fill_config(dh, H, mb, 4, pb, cfg);
    return cfg->lds_bytes <= lds_limit;
}

namespace {

template <int DH, int MB, int NW>
hipError_t launch_one(const FwdArgs& a, const Bf16Config& cfg, hipStream_t s) {
    const int PB = a.m / MB;
    const int units = a.H * PB;
    const int groups = (units + NW - 1) / NW;
    dim3 grid(a.G, groups);
    if (a.norm == 0)
        hipLaunchKernelGGL((sa_bf16_fwd_kernel<DH, MB, NW, false>), grid, dim3(NW * 64), cfg.lds_bytes, s, a, PB,
                           units, cfg.k_row, cfg.v_row);
    else
        hipLaunchKernelGGL((sa_bf16_fwd_kernel<DH, MB, NW, true>), grid, dim3(NW * 64), cfg.lds_bytes, s, a, PB,
                           units, cfg.k_row, cfg.v_row);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_forward(const FwdArgs& a, const Bf16Config& cfg, hipStream_t s) {
    const int dh = a.dh, mb = cfg.protos_per_wave, nw = cfg.waves;
#define SA_CASE(D, M, W) \
    if (dh == D && mb == M && nw == W) return launch_one<D, M, W>(a, cfg, s);
    SA_CASE(32, 16, 4) SA_CASE(32, 32, 4) SA_CASE(32, 64, 4)
    SA_CASE(32, 16, 8) SA_CASE(32, 32, 8) SA_CASE(32, 64, 8)
    SA_CASE(64, 16, 4) SA_CASE(64, 32, 4) SA_CASE(64, 64, 4)
    SA_CASE(64, 16, 8) SA_CASE(64, 32, 8) SA_CASE(64, 64, 8)
    SA_CASE(128, 16, 4) SA_CASE(128, 32, 4)
#undef SA_CASE
    return hipErrorInvalidValue;
}

}  // namespace sa
