// sa_tok_lse.hip -- per-row normaliser of the prototype-axis softmax:
//   lse2[row, h] = log2 sum_j 2^(s[j,row] * scale * log2 e)
// i.e. the denominator of the normalisation display of section 3.1 of the
// SequenceO1 paper, where every history row is allocated across the m
// prototypes.  Rows that are masked or belong to no user get -inf.  The
// forward kernels then weight row i of prototype j by 2^(x - lse2[i]).
#include "sa_internal.h"

namespace sa {

namespace {

// Is buffer row `row` a valid row of some user?
__device__ __forceinline__ bool row_valid(const TokLseArgs& a, int64_t row) {
    if (row >= a.total_rows) return false;
    bool ok;
    if (a.users.cu) {
        ok = row >= a.users.cu[0] && row < a.users.cu[a.users.B];
    } else {
        const int64_t b = row / a.users.L_max, i = row - b * a.users.L_max;
        if (b >= a.users.B) return false;
        const int64_t len = a.users.vcu ? (int64_t)a.users.vcu[b + 1] - a.users.vcu[b] : a.users.L_max;
        ok = i < len;
    }
    if (ok && a.mask) ok = a.mask[row] != 0;
    return ok;
}

__device__ __forceinline__ void lse_merge(float& M, float& Z, float Mo, float Zo) {
    const float Mn = fmaxf(M, Mo);
    if (Mn == -INFINITY) return;
    Z = Z * exp2f(M - Mn) + Zo * exp2f(Mo - Mn);
    M = Mn;
}

}  // namespace

// One wave per 16 rows of one head; S^T[16 rows x 16 prototypes] blocks by MFMA.
template <int DH>
__global__ __launch_bounds__(256) void sa_bf16_tok_lse_kernel(TokLseArgs a) {
    constexpr int KC = DH / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int h = blockIdx.y;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
    if (r0 >= a.total_rows) return;
    const bf16* Kg = (const bf16*)a.K;
    const bf16* Pg = (const bf16*)a.P;

    const int64_t arow = r0 + l16;              // row this lane feeds into the A operand
    const bool aval = row_valid(a, arow);
    bf16x8 ka[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        if (aval) ka[kc] = *(const bf16x8*)(Kg + arow * a.k_stride + (int64_t)h * DH + 32 * kc + 8 * g);
        else ka[kc] = (bf16x8){};
    }
    float M[4], Z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        M[i] = -INFINITY;
        Z[i] = 0.f;
    }
    for (int j0 = 0; j0 < a.m; j0 += 16) {
        const bf16* pr = Pg + ((int64_t)h * a.m + j0 + l16) * DH;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kc], *(const bf16x8*)(pr + 32 * kc + 8 * g), d, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) lse_merge(M[i], Z[i], d[i] * a.c, 1.f);
    }
    // combine the 16 prototype columns held by the 16 lanes of each group
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const float Mo = __shfl_xor(M[i], off, 64);
            const float Zo = __shfl_xor(Z[i], off, 64);
            lse_merge(M[i], Z[i], Mo, Zo);
        }
    }
    if (l16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = r0 + 4 * g + i;
            if (row >= a.total_rows) continue;
            const float v = row_valid(a, row) ? M[i] + log2f(Z[i]) : -INFINITY;
            a.lse2_tok[row * a.H + h] = v;
            if (a.lse_out) a.lse_out[row * a.H + h] = v * kLn2;
        }
    }
}

// fp32: one thread per (row, head), plain FMA.
__global__ __launch_bounds__(256) void sa_f32_tok_lse_kernel(TokLseArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int h = blockIdx.y;
    if (row >= a.total_rows) return;
    float M = -INFINITY, Z = 0.f;
    const bool ok = row_valid(a, row);
    if (ok) {
        const float* Kr = (const float*)a.K + row * a.k_stride + (int64_t)h * a.dh;
        for (int j = 0; j < a.m; ++j) {
            const float* pr = (const float*)a.P + ((int64_t)h * a.m + j) * a.dh;
            float s = 0.f;
            for (int e = 0; e < a.dh; ++e) s = fmaf(pr[e], Kr[e], s);
            lse_merge(M, Z, s * a.c, 1.f);
        }
    }
    const float v = ok ? M + log2f(Z) : -INFINITY;
    a.lse2_tok[row * a.H + h] = v;
    if (a.lse_out) a.lse_out[row * a.H + h] = v * kLn2;
}

hipError_t launch_bf16_tok_lse(const TokLseArgs& a, hipStream_t s) {
    if (a.total_rows == 0) return hipSuccess;
    dim3 grid((unsigned)((a.total_rows + 63) / 64), a.H);
    switch (a.dh) {
        case 32: hipLaunchKernelGGL(sa_bf16_tok_lse_kernel<32>, grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL(sa_bf16_tok_lse_kernel<64>, grid, dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL(sa_bf16_tok_lse_kernel<128>, grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_f32_tok_lse(const TokLseArgs& a, hipStream_t s) {
    if (a.total_rows == 0) return hipSuccess;
    dim3 grid((unsigned)((a.total_rows + 255) / 256), a.H);
    hipLaunchKernelGGL(sa_f32_tok_lse_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
