// sa_gemm.hip -- batched bf16 GEMM with both operands k-contiguous ("NT"):
//     C[z][m][n] = sum_k A[z][m][k] * Bt[z][n][k]        (fp32 accumulation)
// on v_mfma_f32_16x16x32_bf16, for the one-token projections around the STCA
// attention (q = x W_Q before it, (alpha X) W_V after it).
//
// Block = 4 waves = a 128 (m) x 64 (n) tile; wave w owns the 64 x 32 part
// (w / 2, w % 2).  32-wide k-steps of the A and Bt tiles (128 and 64 rows of
// 64 bytes) stream through a 3-stage LDS ring by direct-to-LDS loads, three
// 1 KB loads per wave per stage; the 16-byte chunks of a row are XOR-swizzled
// by (row / 4) % 4 so that a 16-lane operand read touches 16 distinct chunks
// of the 256-byte bank window.  The MFMA computes the transposed tile (A
// operand = Bt rows, B operand = A rows), so a lane's four accumulator rows
// are four consecutive n of one m and its stores are contiguous.  Rows past M
// or N are read from a clamped row and never stored.
#include "sa_device.h"

namespace sa {

using namespace dev;

namespace {

constexpr int kGemmStages = 3;
constexpr int kBM = 128, kBN = 64;
constexpr int kAStage = kBM * 64, kBStage = kBN * 64;    // bytes per stage
constexpr int kOpsPerWave = (kAStage + kBStage) / 1024 / 4;

__device__ __forceinline__ int gemm_swz(int row) { return (row >> 2) & 3; }

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void sa_gemm_nt_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char ring[kGemmStages][kAStage + kBStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int z = blockIdx.z;
    const int bm = blockIdx.x * kBM, bn = blockIdx.y * kBN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 32;
    const bf16* A = a.A + (int64_t)z * a.sA;
    const bf16* Bt = a.Bt + (int64_t)z * a.sB;
    const int ks = a.K / 32;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)&ring[0][0];

    // this lane's part of each of the wave's DMA ops: op o < 8 fills A rows
    // [16 o, 16 o + 16), op o >= 8 fills Bt rows [16 (o - 8), ...); lane ->
    // row + lane / 4, LDS chunk lane % 4 <- logical chunk (lane % 4) ^ swz(row)
    // (the source of a load is the wave-uniform matrix start plus a 32-bit
    // per-lane byte offset; the host keeps both matrices under 4 GB)
    uint32_t voff[kOpsPerWave], dst[kOpsPerWave];
    bool isA[kOpsPerWave];
#pragma unroll
    for (int i = 0; i < kOpsPerWave; ++i) {
        const int o = wave * kOpsPerWave + i;
        isA[i] = o < kBM / 16;
        const int r = 16 * (isA[i] ? o : o - kBM / 16) + lane / 4;
        const int ck = (lane & 3) ^ gemm_swz(r);
        const int64_t grow = isA[i] ? min(bm + r, a.M - 1) : min(bn + r, a.N - 1);
        voff[i] = (uint32_t)((grow * (isA[i] ? a.lda : a.ldb)) * 2 + ck * 16);
        dst[i] = (uint32_t)((isA[i] ? 0 : kAStage) + (isA[i] ? o : o - kBM / 16) * 1024);
    }
    auto issue = [&](int k) {
        const uint32_t base = ring_lds + (uint32_t)((k % kGemmStages) * (kAStage + kBStage));
#pragma unroll
        for (int i = 0; i < kOpsPerWave; ++i)
            dma16c((const unsigned char*)(isA[i] ? (const void*)A : (const void*)Bt) + 64 * k, voff[i],
                   __builtin_amdgcn_readfirstlane(base + dst[i]));
    };

    // operand reads: A rows wm + 16 i + l16 (B operand), Bt rows wn + 16 j + l16 (A operand), chunk g
    uint32_t ra[4], rb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm + 16 * i + l16;
        ra[i] = (uint32_t)(r * 64 + ((g ^ gemm_swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = wn + 16 * j + l16;
        rb[j] = (uint32_t)(kAStage + r * 64 + ((g ^ gemm_swz(r)) * 16));
    }

    f32x4 acc[2][4];   // [n block][m block]: rows n, column m
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int k = 0; k < kGemmStages - 1; ++k)
        if (k < ks) issue(k);
    for (int k = 0; k < ks; ++k) {
        // stage k has landed (own loads), every wave is past stage k - 1
        if (k + 1 < ks) wait_vm<kOpsPerWave>();
        else wait_vm<0>();
        block_barrier();
        if (k + kGemmStages - 1 < ks) issue(k + kGemmStages - 1);
        const uint32_t base = ring_lds + (uint32_t)((k % kGemmStages) * (kAStage + kBStage));
        bf16x8 av[4], bv[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(base + ra[i]);
#pragma unroll
        for (int j = 0; j < 2; ++j) bv[j] = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(base + rb[j]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = mfma(bv[j], av[i], acc[j][i]);
        wait_lgkm0();
    }

    // lane: column m = bm + wm + 16 i + l16, rows n = bn + wn + 16 j + 4 g + 0..3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = bm + wm + 16 * i + l16;
        if (m >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = bn + wn + 16 * j + 4 * g;
            if (n >= a.N) continue;
            const int64_t off = (int64_t)z * a.sC + (int64_t)m * a.ldc + n;
            if constexpr (OUT_BF16) {
                *(bf16x4*)((bf16*)a.C + off) = __builtin_convertvector(acc[j][i], bf16x4);
            } else {
                *(f32x4*)((float*)a.C + off) = acc[j][i];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmArgs& a, bool out_bf16, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0 || a.batch <= 0 || a.K <= 0) return hipSuccess;
    if (a.K % 32 != 0 || a.N % 4 != 0 || (double)a.M * a.lda * 2 >= 4294967296.0 ||
        (double)a.N * a.ldb * 2 >= 4294967296.0)
        return hipErrorInvalidValue;
    dim3 grid((a.M + kBM - 1) / kBM, (a.N + kBN - 1) / kBN, a.batch), block(256);
    if (out_bf16) hipLaunchKernelGGL(sa_gemm_nt_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(sa_gemm_nt_kernel<false>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
