// sa_f32_fwd.hip -- Sketch Attention forward for fp32 inputs with no rounding
// to a narrower type: plain fp32 FMA on the vector ALUs.  It serves small
// fp32 problems (the tiny single-head workload) to fp32 accuracy; bf16 inputs
// take the MFMA kernel.
//
// Block = row range w (same virtual-row segments as the bf16 kernel) x head h
// x up to 256 prototypes; one thread per prototype keeps P_j, the running
// maximum and sum and the dh accumulators in registers, and the block streams
// 32-row tiles of K_h and V_h through LDS.  The online softmax takes the exact
// maximum at every row (history axis, section 3.1 / section 4.4 statistics of
// the SequenceO1 paper); the prototype axis subtracts the per-row normaliser.
#include "sa_internal.h"

namespace sa {

template <int DH>
__global__ __launch_bounds__(256) void sa_f32_fwd_kernel(FwdArgs a) {
    __shared__ float Kt[kTile][DH];
    __shared__ float Vt[kTile][DH];
    __shared__ float Lt[kTile];
    __shared__ int Ok[kTile];
    if (offsets_rejected(a.status)) return;
    const int w = blockIdx.x, h = blockIdx.y;
    const int j = blockIdx.z * 256 + threadIdx.x;
    const bool active = j < a.m;
    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, a.split);
    const int64_t v_lo = rs.lo(w);
    if (v_lo >= total) return;
    const int64_t v_hi = min(rs.lo(w + 1), total);
    const float* Pg = (const float*)a.P;
    const float* Kg = (const float*)a.K;
    const float* Vg = (const float*)a.V;

    float p[DH];
    for (int b = a.users.find(v_lo); b < a.users.B; ++b) {
        const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
        if (us >= v_hi) break;
        const int64_t s_lo = max(v_lo, us), s_hi = min(v_hi, ue);
        if (s_hi <= s_lo) continue;
        if (active) {
            const float* pr = Pg + (int64_t)b * a.q_batch_stride + ((int64_t)h * a.m + j) * DH;
#pragma unroll
            for (int e = 0; e < DH; ++e) p[e] = pr[e];
        }
        const int64_t gbase = a.users.row_base(b) + (s_lo - us);
        const int64_t nrows = s_hi - s_lo;
        float M = -INFINITY, Z = 0.f;
        float acc[DH];
#pragma unroll
        for (int e = 0; e < DH; ++e) acc[e] = 0.f;

        for (int64_t r0 = 0; r0 < nrows; r0 += kTile) {
            const int rows_here = (int)min((int64_t)kTile, nrows - r0);
            __syncthreads();
            for (int x = threadIdx.x; x < kTile * DH; x += 256) {
                const int r = x / DH, e = x - r * DH;
                bool ok = r < rows_here;
                const int64_t grow = gbase + r0 + r;
                if (ok && a.mask) ok = a.mask[grow] != 0;
                Kt[r][e] = ok ? Kg[grow * a.k_stride + (int64_t)h * DH + e] : 0.f;
                Vt[r][e] = ok ? Vg[grow * a.v_stride + (int64_t)h * DH + e] : 0.f;
                if (e == 0) {
                    Ok[r] = ok;
                    Lt[r] = (ok && a.norm == 1) ? a.lse2_tok[grow * a.H + h] : 0.f;
                }
            }
            __syncthreads();
            if (!active) continue;
            for (int r = 0; r < rows_here; ++r) {
                if (!Ok[r]) continue;
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < DH; ++e) s = fmaf(p[e], Kt[r][e], s);
                const float x = s * a.c;
                float wgt;
                if (a.norm == 1) {
                    wgt = exp2f(x - Lt[r]);
                } else {
                    if (x > M) {
                        const float f = exp2f(M - x);   // 0 when M is still -inf
                        Z *= f;
#pragma unroll
                        for (int e = 0; e < DH; ++e) acc[e] *= f;
                        M = x;
                    }
                    wgt = exp2f(x - M);
                    Z += wgt;
                }
#pragma unroll
                for (int e = 0; e < DH; ++e) acc[e] = fmaf(wgt, Vt[r][e], acc[e]);
            }
        }
        if (active) {
            const int64_t base = (((int64_t)w + b) * a.H + h) * a.m + j;
            if (a.norm == 0) {
                a.part.M[base] = M;
                a.part.Z[base] = Z;
            }
#pragma unroll
            for (int e = 0; e < DH; ++e) a.part.acc[base * DH + e] = acc[e];
        }
    }
}

hipError_t launch_f32_forward(const FwdArgs& a, hipStream_t s) {
    dim3 grid(a.G, a.H, (a.m + 255) / 256);
    switch (a.dh) {
        case 16: hipLaunchKernelGGL(sa_f32_fwd_kernel<16>, grid, dim3(256), 0, s, a); break;
        case 32: hipLaunchKernelGGL(sa_f32_fwd_kernel<32>, grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL(sa_f32_fwd_kernel<64>, grid, dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL(sa_f32_fwd_kernel<128>, grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sa
