// issue_rates.hip -- gfx950 issue-rate measurements behind the kernels'
// scheduling choices: per SIMD, how many cycles an MFMA (16x16x32 bf16), a
// v_exp_f32 and a v_fma_f32 take when issued back to back, and what a mix
// costs when the MFMAs and the vector instructions come from one wave or from
// different waves of the same SIMD, and whether a wave's exps and its
// independent FMAs overlap each other; and the LDS read rate per CU for 16-byte
// row reads and 8-byte transposed reads.  One block per CU (256 blocks), w
// waves per SIMD; a block's elapsed shader-clock cycles come from s_memtime
// around the loop (between two barriers), its clock from s_memrealtime
// (100 MHz).  Results are register-only loops or conflict-free LDS reads;
// each thread writes one value so that nothing is optimised away.
//
// Build and run: python -m sketch_attention_flashsa_amd.build --diag, then
// sketch_attention_flashsa_amd/diag/issue_rates (prints one JSON line per
// case).
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kIters = 2048;

enum Mode {
    MFMA = 0, EXP, FMA, MFMA_EXP_SAME, MFMA_FMA_SAME, MFMA_EXP_SPLIT, MFMA_FMA_SPLIT, LDS_B128, LDS_TR_B64,
    EXP_FMA_SAME, MFMA_EXP_FMA_SAME
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

#define EXP8(x) \
    x[0] = __builtin_amdgcn_exp2f(x[0]); x[1] = __builtin_amdgcn_exp2f(x[1]); x[2] = __builtin_amdgcn_exp2f(x[2]); \
    x[3] = __builtin_amdgcn_exp2f(x[3]); x[4] = __builtin_amdgcn_exp2f(x[4]); x[5] = __builtin_amdgcn_exp2f(x[5]); \
    x[6] = __builtin_amdgcn_exp2f(x[6]); x[7] = __builtin_amdgcn_exp2f(x[7]);
#define FMA8(x) \
    for (int i_ = 0; i_ < 8; ++i_) x[i_] = fmaf(x[i_], 1.0001f, 0.5f);
#define MFMA4(c) \
    c[0] = mfma(a, b, c[0]); c[1] = mfma(a, b, c[1]); c[2] = mfma(a, b, c[2]); c[3] = mfma(a, b, c[3]);

template <int MODE>
__global__ void rate_kernel(float* out, long long* cyc, long long* rt, float seed) {
    __shared__ __attribute__((aligned(16))) u32x4 buf[4096];   // 64 KB, for the LDS cases
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (lane + i));
        b[i] = (__bf16)(seed * (lane - i));
    }
    f32x4 c[4];
    for (int i = 0; i < 4; ++i) c[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float x[8], y[8];
    for (int i = 0; i < 8; ++i) {
        x[i] = seed * (lane + i);
        y[i] = seed * (lane - i);
    }
    u32x4 acc4 = {0, 0, 0, 0};
    unsigned s0 = 0, s1 = 0;
    if constexpr (MODE == LDS_B128 || MODE == LDS_TR_B64) {
        for (int i = t; i < 4096; i += blockDim.x) buf[i] = (u32x4){(unsigned)i, 3u * i, 5u * i, 7u * i};
    }
    // waves 4k..4k+3 sit on the four SIMDs; in the split cases odd groups of
    // four run the vector work, even groups the MFMAs
    const bool vec_wave = ((wave >> 2) & 1) != 0;
    __syncthreads();
    const long long c0 = clock64(), r0 = wall_clock64();
    for (int it = 0; it < kIters; ++it) {
        asm volatile("" ::: "memory");
        if constexpr (MODE == MFMA) {
            MFMA4(c)
        } else if constexpr (MODE == EXP) {
            EXP8(x)
        } else if constexpr (MODE == FMA) {
            FMA8(x)
        } else if constexpr (MODE == MFMA_EXP_SAME) {
            c[0] = mfma(a, b, c[0]);
            x[0] = __builtin_amdgcn_exp2f(x[0]); x[1] = __builtin_amdgcn_exp2f(x[1]);
            c[1] = mfma(a, b, c[1]);
            x[2] = __builtin_amdgcn_exp2f(x[2]); x[3] = __builtin_amdgcn_exp2f(x[3]);
            c[2] = mfma(a, b, c[2]);
            x[4] = __builtin_amdgcn_exp2f(x[4]); x[5] = __builtin_amdgcn_exp2f(x[5]);
            c[3] = mfma(a, b, c[3]);
            x[6] = __builtin_amdgcn_exp2f(x[6]); x[7] = __builtin_amdgcn_exp2f(x[7]);
        } else if constexpr (MODE == MFMA_FMA_SAME) {
            c[0] = mfma(a, b, c[0]);
            x[0] = fmaf(x[0], 1.0001f, 0.5f); x[1] = fmaf(x[1], 1.0001f, 0.5f);
            c[1] = mfma(a, b, c[1]);
            x[2] = fmaf(x[2], 1.0001f, 0.5f); x[3] = fmaf(x[3], 1.0001f, 0.5f);
            c[2] = mfma(a, b, c[2]);
            x[4] = fmaf(x[4], 1.0001f, 0.5f); x[5] = fmaf(x[5], 1.0001f, 0.5f);
            c[3] = mfma(a, b, c[3]);
            x[6] = fmaf(x[6], 1.0001f, 0.5f); x[7] = fmaf(x[7], 1.0001f, 0.5f);
        } else if constexpr (MODE == MFMA_EXP_SPLIT) {
            if (vec_wave) {
                EXP8(x)
            } else {
                MFMA4(c)
            }
        } else if constexpr (MODE == MFMA_FMA_SPLIT) {
            if (vec_wave) {
                FMA8(x)
            } else {
                MFMA4(c)
            }
        } else if constexpr (MODE == EXP_FMA_SAME) {
            // eight exps and eight independent FMAs, alternating (the
            // scheduling barriers keep that order)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = __builtin_amdgcn_exp2f(x[i]);
                y[i] = fmaf(y[i], 1.0001f, 0.5f);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (MODE == MFMA_EXP_FMA_SAME) {
            // four MFMAs, each followed by two exps and two independent FMAs
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = mfma(a, b, c[i]);
                x[2 * i] = __builtin_amdgcn_exp2f(x[2 * i]);
                y[2 * i] = fmaf(y[2 * i], 1.0001f, 0.5f);
                x[2 * i + 1] = __builtin_amdgcn_exp2f(x[2 * i + 1]);
                y[2 * i + 1] = fmaf(y[2 * i + 1], 1.0001f, 0.5f);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (MODE == LDS_B128) {
            // 8 reads of 64 lanes x 16 consecutive bytes (1 KB each)
            const int base = ((it + wave) & 7) * 512;
#pragma unroll
            for (int k = 0; k < 8; k += 2) {
                const u32x4 p = buf[(base + k * 64 + lane) & 4095];
                const u32x4 q = buf[(base + (k + 1) * 64 + lane) & 4095];
                acc4 = acc4 + p + q;
            }
        } else {
            // 16 transposed reads of 64 lanes x 8 bytes (512 B each)
            const int base = ((it + wave) & 7) * 1024;
            lds_i16x4* p0 = (lds_i16x4*)(uintptr_t)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&buf[0];
#pragma unroll
            for (int k = 0; k < 16; k += 2) {
                const u32x2 p = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0 + ((base + k * 64 + lane) & 8191)));
                const u32x2 q = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0 + ((base + (k + 1) * 64 + lane) & 8191)));
                s0 += p[0] + q[0];
                s1 += p[1] + q[1];
            }
        }
    }
    __syncthreads();
    const long long c1 = clock64(), r1 = wall_clock64();
    float r = c[0][0] + c[1][1] + c[2][2] + c[3][3];
    for (int i = 0; i < 8; ++i) r += x[i] + y[i];
    r += (float)(acc4[0] ^ acc4[1] ^ acc4[2] ^ acc4[3] ^ s0 ^ s1);
    out[blockIdx.x * blockDim.x + t] = r;
    if (t == 0) {
        cyc[blockIdx.x] = c1 - c0;
        rt[blockIdx.x] = r1 - r0;
    }
}

struct Case {
    const char* name;
    int mode;
    int mfma, exp, fma;        // per wave-iteration of an MFMA-issuing / vector wave
    double lds_bytes;          // per wave-iteration
    bool split;
};

template <int MODE>
void run(const Case& cs, int wps) {
    const int blocks = 256, threads = 256 * wps;
    float* out;
    long long *cyc, *rt;
    if (hipMalloc(&out, sizeof(float) * blocks * threads) != hipSuccess || hipMalloc(&cyc, 8 * blocks) != hipSuccess ||
        hipMalloc(&rt, 8 * blocks) != hipSuccess) {
        printf("{\"error\": \"hipMalloc\"}\n");
        return;
    }
    for (int rep = 0; rep < 2; ++rep) hipLaunchKernelGGL(rate_kernel<MODE>, dim3(blocks), dim3(threads), 0, 0, out, cyc, rt, 0.001f);
    hipDeviceSynchronize();
    long long hc[256], hr[256];
    hipMemcpy(hc, cyc, sizeof(hc), hipMemcpyDeviceToHost);
    hipMemcpy(hr, rt, sizeof(hr), hipMemcpyDeviceToHost);
    double c = 0, r = 0;
    for (int i = 0; i < blocks; ++i) {
        c += hc[i];
        r += hr[i];
    }
    c /= blocks;
    r /= blocks;
    // per SIMD: wps waves, each kIters iterations (in split cases half of them
    // MFMA waves, half vector waves)
    const double iters = (double)kIters * wps;
    const double mf = cs.split ? iters / 2 * cs.mfma : iters * cs.mfma;
    const double vv = cs.split ? iters / 2 * (cs.exp + cs.fma) : iters * (cs.exp + cs.fma);
    printf("{\"case\": \"%s\", \"waves_per_simd\": %d, \"cycles\": %.0f, \"clock_mhz\": %.0f, "
           "\"mfma_per_simd\": %.0f, \"vector_per_simd\": %.0f, \"cycles_per_simd_iteration\": %.2f",
           cs.name, wps, c, c / (r / 100.0), mf, vv, c / iters);
    if (cs.lds_bytes > 0) printf(", \"lds_bytes_per_cycle_per_cu\": %.1f", cs.lds_bytes * iters * 4 / c);
    printf("}\n");
    hipFree(out);
    hipFree(cyc);
    hipFree(rt);
}

int main() {
    const Case cases[] = {
        {"mfma_16x16x32_bf16 x4", MFMA, 4, 0, 0, 0, false},
        {"v_exp_f32 x8", EXP, 0, 8, 0, 0, false},
        {"v_fma_f32 x8", FMA, 0, 0, 8, 0, false},
        {"mfma x4 + exp x8, one wave", MFMA_EXP_SAME, 4, 8, 0, 0, false},
        {"mfma x4 + fma x8, one wave", MFMA_FMA_SAME, 4, 0, 8, 0, false},
        {"mfma x4 waves + exp x8 waves (split)", MFMA_EXP_SPLIT, 4, 8, 0, 0, true},
        {"mfma x4 waves + fma x8 waves (split)", MFMA_FMA_SPLIT, 4, 0, 8, 0, true},
        {"ds_read_b128 x8", LDS_B128, 0, 0, 0, 8 * 1024.0, false},
        {"ds_read_b64_tr_b16 x16", LDS_TR_B64, 0, 0, 0, 16 * 512.0, false},
        {"exp x8 + fma x8, one wave", EXP_FMA_SAME, 0, 8, 8, 0, false},
        {"mfma x4 + exp x8 + fma x8, one wave", MFMA_EXP_FMA_SAME, 4, 8, 8, 0, false},
    };
    for (int wps : {1, 2, 4}) {
        for (const Case& cs : cases) {
            if (cs.split && wps < 2) continue;
            switch (cs.mode) {
                case MFMA: run<MFMA>(cs, wps); break;
                case EXP: run<EXP>(cs, wps); break;
                case FMA: run<FMA>(cs, wps); break;
                case MFMA_EXP_SAME: run<MFMA_EXP_SAME>(cs, wps); break;
                case MFMA_FMA_SAME: run<MFMA_FMA_SAME>(cs, wps); break;
                case MFMA_EXP_SPLIT: run<MFMA_EXP_SPLIT>(cs, wps); break;
                case MFMA_FMA_SPLIT: run<MFMA_FMA_SPLIT>(cs, wps); break;
                case LDS_B128: run<LDS_B128>(cs, wps); break;
                case EXP_FMA_SAME: run<EXP_FMA_SAME>(cs, wps); break;
                case MFMA_EXP_FMA_SAME: run<MFMA_EXP_FMA_SAME>(cs, wps); break;
                default: run<LDS_TR_B64>(cs, wps); break;
            }
        }
    }
    return 0;
}
