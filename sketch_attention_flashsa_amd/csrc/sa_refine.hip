// sa_refine.hip -- the per-layer sketch update of stacked Sketch Attention
// refinement (section 3.3 of the SequenceO1 paper): after a layer's
// attention pass has produced Xhat = A X for every user, each sketch row
// (user b, prototype j) of width D = H*dh becomes
//     Xbar = LN1(Xt + Xhat),   Xt' = LN2(Xbar + (silu(Xbar W1) * (Xbar W3)) W2),
// and, when another layer follows, that layer's queries Q' = Xt' Wq' (bf16,
// [B, H, m, dh], the layout the attention kernels read).  The FFN is the
// paper's sketch SwiGLU with inner width F = 2D (appendix G).
//
// One block = 128 sketch rows, 8 waves; wave w owns rows 16w..16w+15 through
// every phase:
//   A  LN1 computed directly in the MFMA A-operand layout (the four lanes of
//      a row hold D/4 of its features each; two shuffles reduce a row), Xbar
//      kept in fp32 in the output rows (overwritten in D) and as bf16
//      operands in registers;
//   B  [a | g] = Xbar [W1 | W3] on v_mfma_f32_16x16x32_bf16, 32 hidden units
//      at a time, h = silu(a) * g through a small per-wave LDS chunk (bf16)
//   C  into f += h W2 for those units; the weights of the next 32 units are
//      loaded into registers while a chunk is computed and stored into the
//      other half of a double-buffered LDS stage, so the 8 waves share each
//      weight byte (the hidden layer never exists whole);
//   D  z = Xbar + f, LN2 per row (lane-group reductions), fp32 out;
//   E  optional Q' = Xt' Wq' on MFMA, bf16 out.
// The projection-only mode runs E alone on fp32 input rows (the first
// layer's queries P0 Wq).  Weight matrices arrive transposed ([out][in], made
// by sa_transpose_kernel from the [in][out] arguments) so that every MFMA B
// operand is one 16-byte read.
#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kRows = 128;       // sketch rows per block (8 waves x 16)

// sum over the 16 lanes that share l / 16
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float silu(float a) {
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * kLog2e));
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512, 2) void sa_sketch_kernel(SketchArgs a) {
    constexpr int F = 2 * D;
    constexpr int KS = D / 32;           // k-steps over the D features
    constexpr int NCB = D / 16;          // 16-column blocks of a D-wide output
    constexpr int WR = D + 8;            // LDS row stride of a [32][D] weight chunk (elements)
    constexpr int W2R = 32 + 8;          // LDS row stride of a [D][32] weight chunk
    constexpr int CH = 2 * 32 * WR + D * W2R;   // elements of one FFN chunk (W1, W3, W2 parts)
    constexpr int PER = 12 * D / 512;    // 16-byte pieces of one chunk per thread
    static_assert(PER * 512 == 12 * D, "whole pieces per thread");
    __shared__ __attribute__((aligned(16))) bf16 wbuf[2][CH];
    __shared__ __attribute__((aligned(16))) bf16 hch[8][16 * W2R];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int r0 = blockIdx.x * kRows + 16 * wave;   // this wave's first row
    // A-operand layout: lane (l16, g) holds row r0 + l16, features 32 ks + 8 g + j
    const int ra = r0 + l16;
    const bool rok = ra < a.rows;

    // ---- the FFN weights stream through LDS in chunks of 32 hidden units:
    // W1^T and W3^T rows [n0, n0 + 32) and W2^T columns [n0, n0 + 32)
    bf16x8 pre[PER];
    auto piece = [&](int idx, int n0, const bf16*& src, int& dst) {
        // idx < 4 D: W1 part, < 8 D: W3 part, else W2 part
        if (idx < 8 * D) {
            const int part = idx / (4 * D), k = idx - part * 4 * D;
            const int u = k / (D / 8), c8 = k - u * (D / 8);
            src = (part == 0 ? a.w1t : a.w3t) + (size_t)(n0 + u) * D + c8 * 8;
            dst = part * 32 * WR + u * WR + c8 * 8;
        } else {
            const int k = idx - 8 * D, r = k >> 2, c8 = k & 3;
            src = a.w2t + (size_t)r * F + n0 + c8 * 8;
            dst = 2 * 32 * WR + r * W2R + c8 * 8;
        }
    };
    auto load_chunk = [&](int n0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const bf16* src;
            int dst;
            piece(threadIdx.x + u * 512, n0, src, dst);
            pre[u] = *(const bf16x8*)src;
        }
    };
    auto store_chunk = [&](int buf, int n0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const bf16* src;
            int dst;
            piece(threadIdx.x + u * 512, n0, src, dst);
            *(bf16x8*)&wbuf[buf][dst] = pre[u];
        }
    };

    bf16x8 af[KS];
    if (a.mode == 1) {
        // projection only: fp32 rows (the prototypes) straight into A operands
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = rok ? a.base[(size_t)ra * D + 32 * ks + 8 * g + j] : 0.f;
            af[ks] = cat8(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
        }
    } else {
        load_chunk(0);
        // ---- A: y = Xt + Xhat and Xbar = LN1(y), in the A-operand layout: the
        // four lanes of a row (g = 0..3) hold D/4 features each
        const int b = rok ? ra / a.m : 0, jr = rok ? ra - b * a.m : 0;
        const float* brow = a.base + (size_t)(a.base_shared ? jr : ra) * D;
        float y[KS][8];
        float sm = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // features 32 ks + 8 g + j: head ks (dh = 32), element 8 g + j
            const float* xr = a.xhat + (((size_t)b * a.H + ks) * a.m + jr) * 32 + 8 * g;
            const f32x4 x0 = rok ? *(const f32x4*)xr : (f32x4){0.f, 0.f, 0.f, 0.f};
            const f32x4 x1 = rok ? *(const f32x4*)(xr + 4) : (f32x4){0.f, 0.f, 0.f, 0.f};
            const f32x4 b0 = rok ? *(const f32x4*)(brow + 32 * ks + 8 * g) : (f32x4){0.f, 0.f, 0.f, 0.f};
            const f32x4 b1 = rok ? *(const f32x4*)(brow + 32 * ks + 8 * g + 4) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y[ks][j] = b0[j] + x0[j];
                y[ks][4 + j] = b1[j] + x1[j];
                sm += y[ks][j] + y[ks][4 + j];
            }
        }
        sm += __shfl_xor(sm, 16, 64);
        sm += __shfl_xor(sm, 32, 64);
        const float mean = sm * (1.0f / D);
        float q = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) q += (y[ks][j] - mean) * (y[ks][j] - mean);
        q += __shfl_xor(q, 16, 64);
        q += __shfl_xor(q, 32, 64);
        const float inv = 1.0f / sqrtf(q * (1.0f / D) + a.eps);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * ks + 8 * g + j;
                x[j] = rok ? (y[ks][j] - mean) * inv * a.ln1_g[c] + a.ln1_b[c] : 0.f;
            }
            if (rok) {
                // kept in fp32 for the second residual (read back in the output layout)
                *(f32x4*)(a.out + (size_t)ra * D + 32 * ks + 8 * g) = (f32x4){x[0], x[1], x[2], x[3]};
                *(f32x4*)(a.out + (size_t)ra * D + 32 * ks + 8 * g + 4) = (f32x4){x[4], x[5], x[6], x[7]};
            }
            af[ks] = cat8(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
        }
        store_chunk(0, 0);
        __syncthreads();

        // ---- B, C: per chunk, a = Xbar W1 and g = Xbar W3 (16 rows x 32 units),
        // h = silu(a) * g through this wave's LDS chunk into the A operand,
        // f += h W2[chunk rows]; chunk c + 1 is loaded while c is computed
        f32x4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        bf16* hw = hch[wave];
        for (int c = 0; c < F / 32; ++c) {
            const int cur = c & 1;
            const bool more = c + 1 < F / 32;
            if (more) load_chunk(32 * (c + 1));
            const bf16* w1s = wbuf[cur];
            const bf16* w3s = wbuf[cur] + 32 * WR;
            const bf16* w2s = wbuf[cur] + 2 * 32 * WR;
            f32x4 ga[2], gg[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) ga[cb] = gg[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    ga[cb] = mfma(af[ks], *(const bf16x8*)&w1s[(16 * cb + l16) * WR + 32 * ks + 8 * g], ga[cb]);
                    gg[cb] = mfma(af[ks], *(const bf16x8*)&w3s[(16 * cb + l16) * WR + 32 * ks + 8 * g], gg[cb]);
                }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) hw[(4 * g + i) * W2R + 16 * cb + l16] = (bf16)(silu(ga[cb][i]) * gg[cb][i]);
            const bf16x8 hf = *(const bf16x8*)&hw[l16 * W2R + 8 * g];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                acc[cb] = mfma(hf, *(const bf16x8*)&w2s[(16 * cb + l16) * W2R + 8 * g], acc[cb]);
            if (more) store_chunk(cur ^ 1, 32 * (c + 1));
            __syncthreads();
        }

        // ---- D: Xt' = LN2(Xbar + f); row r0 + 4g + i lives in the 16 lanes of
        // group g, one feature per column block
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 4 * g + i;
            const bool ok = r < a.rows;
            float z[NCB];
            float s2 = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                z[cb] = acc[cb][i] + (ok ? a.out[(size_t)r * D + 16 * cb + l16] : 0.f);
                s2 += z[cb];
            }
            const float mean2 = group16_sum(s2) * (1.0f / D);
            float q2 = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) q2 += (z[cb] - mean2) * (z[cb] - mean2);
            const float inv2 = 1.0f / sqrtf(group16_sum(q2) * (1.0f / D) + a.eps);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int cc = 16 * cb + l16;
                if (ok) a.out[(size_t)r * D + cc] = (z[cb] - mean2) * inv2 * a.ln2_g[cc] + a.ln2_b[cc];
            }
        }
        if (!a.wqt) return;
        // the new rows, back in the A-operand layout
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = rok ? a.out[(size_t)ra * D + 32 * ks + 8 * g + j] : 0.f;
            af[ks] = cat8(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
        }
    }

    // ---- E: Q' = Xt' Wq' (bf16, [B][H][m][dh]), Wq'^T read from memory (it is
    // shared by every block and stays in L2)
    if (a.wqt) {
#pragma unroll 1
        for (int n0 = 0; n0 < D; n0 += 64) {
            f32x4 acc[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[cb] = mfma(af[ks], *(const bf16x8*)(a.wqt + (size_t)(n0 + 16 * cb + l16) * D + 32 * ks + 8 * g),
                                   acc[cb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 4 * g + i;
                if (r >= a.rows) continue;
                const int b = r / a.m, j = r - b * a.m;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int c = n0 + 16 * cb + l16, h = c / a.dh, e = c - h * a.dh;
                    a.q[(((size_t)b * a.H + h) * a.m + j) * a.dh + e] = (bf16)acc[cb][i];
                }
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
    const dim3 grid((a.rows + kRows - 1) / kRows), block(512);
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
