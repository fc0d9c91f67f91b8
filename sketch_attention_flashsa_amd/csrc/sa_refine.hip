// sa_refine.hip -- the per-layer sketch update of stacked Sketch Attention
// refinement (section 3.3 of the SequenceO1 paper): after a layer's
// attention pass has produced Xhat = A X for every user, each sketch row
// (user b, prototype j) of width D = H*dh becomes
//     Xbar = LN1(Xt + Xhat),   Xt' = LN2(Xbar + (silu(Xbar W1) * (Xbar W3)) W2),
// and, when another layer follows, that layer's queries Q' = Xt' Wq' (bf16,
// [B, H, m, dh], the layout the attention kernels read).  The FFN is the
// paper's sketch SwiGLU with inner width F = 2D (appendix G).
//
// One block = 64 sketch rows, 4 waves; wave w owns rows 16w..16w+15 through
// every phase, so the only block barrier is after the first one:
//   A  LN1 per row (lanes across the D features, fp32), Xbar kept in fp32 in
//      the output rows (overwritten in D) and in bf16 in LDS;
//   B  [a | g] = Xbar [W1 | W3] on v_mfma_f32_16x16x32_bf16, 64 hidden units
//      at a time, h = silu(a) * g through a small per-wave LDS chunk (bf16)
//   C  into f += h W2 for those 64 units, so the hidden layer never exists
//      whole (43 KB of LDS per block);
//   D  z = Xbar + f, LN2 per row (lane-group reductions), fp32 out;
//   E  optional Q' = Xt' Wq' on MFMA, bf16 out.
// The projection-only mode runs E alone on fp32 input rows (the first
// layer's queries P0 Wq).  Weight matrices arrive transposed ([out][in], made
// by sa_transpose_kernel from the [in][out] arguments) so that every MFMA B
// operand is one 16-byte load; they are shared by all blocks and stay in L2.
#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kRows = 64;        // sketch rows per block

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
// sum over the 16 lanes that share l / 16
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float silu(float a) {
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * kLog2e));
}

// acc[cb] (16 rows x 16 columns each) += A x B over KS k-steps of 32: A row
// l16 of this lane group starts at `a_row` (LDS, k contiguous); B column
// 16 cb + l16 is row 16 cb + l16 of the transposed weight `wt` (k
// contiguous, `ldw` elements between rows).
template <int KS, int NCB>
__device__ __forceinline__ void gemm_rows16(f32x4 (&acc)[NCB], const bf16* a_row, const bf16* __restrict__ wt,
                                            int ldw, int l16, int g) {
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *(const bf16x8*)(a_row + 32 * ks + 8 * g);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const bf16x8 bw = *(const bf16x8*)(wt + (size_t)(16 * cb + l16) * ldw + 32 * ks + 8 * g);
            acc[cb] = mfma(a, bw, acc[cb]);
        }
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void sa_sketch_kernel(SketchArgs a) {
    constexpr int F = 2 * D;
    constexpr int XS = D + 8;          // bf16 row strides in LDS (16-byte aligned rows, shifted banks)
    constexpr int HC = 64 + 8;         // one 64-unit chunk of the hidden layer
    constexpr int VEC = D / 64;        // features per lane in the row-wise phases
    constexpr int NCB = D / 16;        // 16-column blocks of a D-wide output
    __shared__ __attribute__((aligned(16))) bf16 xb[kRows * XS];
    __shared__ __attribute__((aligned(16))) bf16 hch[4 * 16 * HC];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int tile0 = blockIdx.x * kRows;
    const int wrow0 = 16 * wave;                     // this wave's first row in the tile
    const int c0 = lane * VEC;                        // row-wise phases: this lane's features

    if (a.mode == 1) {
        // projection only: fp32 rows -> bf16 in LDS
        for (int t = 0; t < 16; ++t) {
            const int rl = wrow0 + t, r = tile0 + rl;
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                xb[rl * XS + c0 + v] = (bf16)(r < a.rows ? a.base[(size_t)r * D + c0 + v] : 0.f);
        }
    } else {
        // ---- A: y = Xt + Xhat, Xbar = LN1(y)
        for (int t = 0; t < 16; ++t) {
            const int rl = wrow0 + t, r = tile0 + rl;
            if (r >= a.rows) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) xb[rl * XS + c0 + v] = (bf16)0.f;
                continue;
            }
            const int b = r / a.m, j = r - b * a.m;
            const float* brow = a.base_shared ? a.base + (size_t)j * D : a.base + (size_t)r * D;
            const int h = c0 / a.dh, e = c0 - h * a.dh;
            const float* xrow = a.xhat + (((size_t)b * a.H + h) * a.m + j) * a.dh + e;
            float y[VEC];
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                y[v] = brow[c0 + v] + xrow[v];
                s += y[v];
            }
            const float mean = wave_sum(s) * (1.0f / D);
            float q = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) q += (y[v] - mean) * (y[v] - mean);
            const float inv = 1.0f / sqrtf(wave_sum(q) * (1.0f / D) + a.eps);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float xbar = (y[v] - mean) * inv * a.ln1_g[c0 + v] + a.ln1_b[c0 + v];
                a.out[(size_t)r * D + c0 + v] = xbar;       // kept for the second residual
                xb[rl * XS + c0 + v] = (bf16)xbar;
            }
        }
        // the fp32 Xbar rows are read back in another lane order in D
        __syncthreads();

        // ---- B, C: per chunk of 64 hidden units, a = Xbar W1 and g = Xbar W3
        // (16 rows x 64 each), h = silu(a) * g through this wave's LDS chunk
        // into the A operand, f += h W2[chunk rows]
        const bf16* arow = xb + (wrow0 + l16) * XS;
        bf16* hw = hch + wave * 16 * HC;
        f32x4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int n0 = 0; n0 < F; n0 += 64) {
            f32x4 acc_a[4], acc_g[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc_a[cb] = acc_g[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
            gemm_rows16<D / 32, 4>(acc_a, arow, a.w1t + (size_t)n0 * D, D, l16, g);
            gemm_rows16<D / 32, 4>(acc_g, arow, a.w3t + (size_t)n0 * D, D, l16, g);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hw[(4 * g + i) * HC + 16 * cb + l16] = (bf16)(silu(acc_a[cb][i]) * acc_g[cb][i]);
            gemm_rows16<2, NCB>(acc, hw + l16 * HC, a.w2t + n0, F, l16, g);
        }

        // ---- D: Xt' = LN2(Xbar + f); row 4g + i of the wave lives in the 16
        // lanes of group g, 16 features per lane (one per column block)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = wrow0 + 4 * g + i, r = tile0 + rl;
            const bool ok = r < a.rows;
            float z[NCB];
            float s = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                z[cb] = acc[cb][i] + (ok ? a.out[(size_t)r * D + 16 * cb + l16] : 0.f);
                s += z[cb];
            }
            const float mean = group16_sum(s) * (1.0f / D);
            float q = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) q += (z[cb] - mean) * (z[cb] - mean);
            const float inv = 1.0f / sqrtf(group16_sum(q) * (1.0f / D) + a.eps);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int c = 16 * cb + l16;
                const float o = (z[cb] - mean) * inv * a.ln2_g[c] + a.ln2_b[c];
                if (ok) a.out[(size_t)r * D + c] = o;
                xb[rl * XS + c] = (bf16)(ok ? o : 0.f);
            }
        }
    }

    // ---- E: Q' = Xt' Wq' (bf16, [B][H][m][dh])
    if (a.wqt) {
        f32x4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        gemm_rows16<D / 32, NCB>(acc, xb + (wrow0 + l16) * XS, a.wqt, D, l16, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = tile0 + wrow0 + 4 * g + i;
            if (r >= a.rows) continue;
            const int b = r / a.m, j = r - b * a.m;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int c = 16 * cb + l16, h = c / a.dh, e = c - h * a.dh;
                a.q[(((size_t)b * a.H + h) * a.m + j) * a.dh + e] = (bf16)acc[cb][i];
            }
        }
    }
}

// dst[c][r] = src[r][c] for up to kMaxTranspose bf16 matrices (blockIdx.z),
// 32 x 32 tiles through LDS.
__global__ __launch_bounds__(256) void sa_transpose_kernel(TransposeArgs a) {
    const TransposeArgs::Mat& t = a.mat[blockIdx.z];
    __shared__ bf16 tile[32][33];
    const int r0 = blockIdx.y * 32, cc0 = blockIdx.x * 32;
    if (r0 >= t.rows || cc0 >= t.cols) return;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;     // 32 x 8
    for (int k = ty; k < 32; k += 8) {
        const int r = r0 + k, c = cc0 + tx;
        tile[k][tx] = (r < t.rows && c < t.cols) ? t.src[(size_t)r * t.cols + c] : (bf16)0.f;
    }
    __syncthreads();
    for (int k = ty; k < 32; k += 8) {
        const int c = cc0 + k, r = r0 + tx;
        if (c < t.cols && r < t.rows) t.dst[(size_t)c * t.rows + r] = tile[tx][k];
    }
}

bool sketch_supported(int D) { return D == 128 || D == 256; }

hipError_t launch_sketch(const SketchArgs& a, int D, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const dim3 grid((a.rows + kRows - 1) / kRows), block(256);
    if (D == 128) hipLaunchKernelGGL(sa_sketch_kernel<128>, grid, block, 0, s, a);
    else if (D == 256) hipLaunchKernelGGL(sa_sketch_kernel<256>, grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    int mr = 1, mc = 1;
    for (int i = 0; i < a.n; ++i) {
        mr = a.mat[i].rows > mr ? a.mat[i].rows : mr;
        mc = a.mat[i].cols > mc ? a.mat[i].cols : mc;
    }
    hipLaunchKernelGGL(sa_transpose_kernel, dim3((mc + 31) / 32, (mr + 31) / 32, a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa

namespace sa {

using namespace dev;

// Row projection out = X W for the fused entry's two-pass shapes: X [rows][DIN]
// bf16 (row stride x_stride), W^T [NOUT][DIN] bf16 (transposed weights, staged
// in LDS once per block), out [rows][NOUT] bf16.  16 waves, 16 rows each per
// pass over a 256-row tile; A operands straight from memory (16 bytes per
// lane), B operands from LDS, v_mfma_f32_16x16x32_bf16.
template <int DIN, int NOUT>
__global__ __launch_bounds__(1024) void sa_project_kernel(ProjectArgs a) {
    constexpr int WS = DIN + 8;
    constexpr int NCB = 8;                     // 128 output columns per pass
    __shared__ __attribute__((aligned(16))) bf16 wl[NOUT * WS];
    for (int i = threadIdx.x; i < NOUT * DIN / 8; i += 1024) {
        const int r = i / (DIN / 8), c8 = i - r * (DIN / 8);
        *(bf16x8*)&wl[r * WS + c8 * 8] = *(const bf16x8*)(a.wt + (size_t)r * DIN + c8 * 8);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    for (int64_t t0 = (int64_t)blockIdx.x * 256; t0 < a.rows; t0 += (int64_t)gridDim.x * 256) {
        const int64_t r0 = t0 + 16 * wave;
        if (r0 >= a.rows) continue;
        const int64_t ra = min(r0 + l16, a.rows - 1);
#pragma unroll 1
        for (int n0 = 0; n0 < NOUT; n0 += 128) {
            f32x4 acc[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DIN / 32; ++ks) {
                const bf16x8 x = *(const bf16x8*)(a.X + ra * a.x_stride + 32 * ks + 8 * g);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    acc[cb] = mfma(x, *(const bf16x8*)&wl[(n0 + 16 * cb + l16) * WS + 32 * ks + 8 * g], acc[cb]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + 4 * g + i;
                if (r >= a.rows) continue;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) a.out[r * NOUT + n0 + 16 * cb + l16] = (bf16)acc[cb][i];
            }
        }
    }
}

bool project_supported(int din, int nout) { return (din == 128 || din == 256) && (nout == 128 || nout == 256); }

hipError_t launch_project(const ProjectArgs& a, int din, int nout, int grid, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const int64_t tiles = (a.rows + 255) / 256;
    const dim3 gr((unsigned)(tiles < grid ? tiles : grid)), blk(1024);
    if (din == 128 && nout == 128) hipLaunchKernelGGL((sa_project_kernel<128, 128>), gr, blk, 0, s, a);
    else if (din == 128 && nout == 256) hipLaunchKernelGGL((sa_project_kernel<128, 256>), gr, blk, 0, s, a);
    else if (din == 256 && nout == 128) hipLaunchKernelGGL((sa_project_kernel<256, 128>), gr, blk, 0, s, a);
    else if (din == 256 && nout == 256) hipLaunchKernelGGL((sa_project_kernel<256, 256>), gr, blk, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sa
