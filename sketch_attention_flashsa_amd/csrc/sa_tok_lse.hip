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

// bf16: one wave per head (4 heads per block; blocks of the same rows for
// the other heads are dispatched next to it, so every row is read while it is
// in the caches), walking 32-row tiles with the next tile's key fragments
// loaded while the current one is computed.  The wave keeps P for up to 128
// prototypes in registers (A operands, one 16-prototype block per sb); each
// 16-row half gives S [16 sb prototypes x 16 rows] by MFMA, a lane holding
// prototypes 16 sb + 4 g + i of row l16: the row maximum and the sum of
// 2^(s c - max) take the lane's 4 NSB values, then the 4 lanes of the row
// (one exponential per score, two shuffles per reduction).  More than 128
// prototypes are taken 128 at a time with a running (max, sum) merge.
template <int DH>
__global__ __launch_bounds__(256) void sa_bf16_tok_lse_kernel(TokLseArgs a) {
    constexpr int KC = DH / 32;
    constexpr int NSB = 8;                        // 16-prototype blocks held at a time
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int h = blockIdx.x * 4 + wave;
    if (h >= a.H) return;
    const int64_t ntile = (a.total_rows + 31) / 32;
    if (offsets_rejected(a.status)) {
        // offsets failed the check: no key is read, the row normalisers are NaN
        for (int64_t t = blockIdx.y; t < ntile; t += gridDim.y) {
            const int64_t row = 32 * t + (lane & 31);
            if (lane < 32 && row < a.total_rows && a.lse_out) a.lse_out[row * a.H + h] = __builtin_nanf("");
        }
        return;
    }
    const bf16* Kg = (const bf16*)a.K + (int64_t)h * DH + 8 * g;
    const bf16* Pg = (const bf16*)a.P + (int64_t)h * a.m * DH + 8 * g;
    const int nchunk = (a.m + 16 * NSB - 1) / (16 * NSB);

    // key fragments of tile t: B operands, column = row 32 t + 16 half + l16 (clamped), k = dh
    auto load_k = [&](int64_t t, bf16x8 (&kf)[2][KC]) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t row = min(32 * t + 16 * half + l16, a.total_rows - 1);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) kf[half][kc] = *(const bf16x8*)(Kg + row * a.k_stride + 32 * kc);
        }
    };
    // prototype fragments: A operands, row = prototype 16 sb + l16 (clamped), k = dh
    bf16x8 pf[NSB][KC];
    auto load_p = [&](int c) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int j = min(16 * (NSB * c + sb) + l16, a.m - 1);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) pf[sb][kc] = *(const bf16x8*)(Pg + (int64_t)j * DH + 32 * kc);
        }
    };
    if (nchunk == 1) load_p(0);

    int64_t t = blockIdx.y;
    bf16x8 kf[2][KC], kn[2][KC];
    if (t < ntile) load_k(t, kf);
    for (; t < ntile; t += gridDim.y) {
        const bool more = t + gridDim.y < ntile;
        if (more) load_k(t + gridDim.y, kn);
        float M[2] = {-INFINITY, -INFINITY}, Z[2] = {0.f, 0.f};
        for (int c = 0; c < nchunk; ++c) {
            if (nchunk > 1) load_p(c);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float x[NSB][4];
                float mx = -INFINITY;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc)
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[sb][kc], kf[half][kc], sc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool ok = 16 * (NSB * c + sb) + 4 * g + i < a.m;
                        x[sb][i] = ok ? sc[i] * a.c : -INFINITY;
                        mx = fmaxf(mx, x[sb][i]);
                    }
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                float z = 0.f;
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) z += __builtin_amdgcn_exp2f(x[sb][i] - mx);
                z += __shfl_xor(z, 16, 64);
                z += __shfl_xor(z, 32, 64);
                lse_merge(M[half], Z[half], mx, z);
            }
        }
        // lanes of group 0 write the 16 rows of each half
        if (g == 0) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int64_t row = 32 * t + 16 * half + l16;
                if (row < a.total_rows) {
                    const float v = row_valid(a, row) ? M[half] + log2f(Z[half]) : -INFINITY;
                    a.lse2_tok[row * a.H + h] = v;
                    if (a.lse_out) a.lse_out[row * a.H + h] = v * kLn2;
                }
            }
        }
        if (more) {
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) kf[half][kc] = kn[half][kc];
        }
    }
}

// fp32: one thread per (row, head), plain FMA.
__global__ __launch_bounds__(256) void sa_f32_tok_lse_kernel(TokLseArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int h = blockIdx.y;
    if (row >= a.total_rows) return;
    if (offsets_rejected(a.status)) {
        if (a.lse_out) a.lse_out[row * a.H + h] = __builtin_nanf("");
        return;
    }
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
    // x: groups of 4 heads (the blocks of one row range run side by side), y:
    // row tiles, strided; a few waves per SIMD of work per CU
    const int64_t ntile = (a.total_rows + 31) / 32;
    const int hg = (a.H + 3) / 4;
    const int64_t want = (int64_t)2048 / hg;          // ~8 blocks per CU on 256 CUs
    dim3 grid((unsigned)hg, (unsigned)(ntile < want ? ntile : want));
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
