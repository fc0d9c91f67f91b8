// sa_merge.hip -- second pass of the split-row Sketch Attention forward, and
// the prefix of dense lengths that places users on the virtual row axis.
//
// History axis: every segment (w, b) left (M_w, Z_w, acc_w) with
//   Z_w = sum_i 2^(x_i - M_w),  acc_w = sum_i 2^(x_i - M_w) V_i,  x = s*scale*log2(e).
// User b's sketch is the log-sum-exp combination over its segments in
// ascending w (the max and log-sum-exp statistics of section 4.4 of the
// SequenceO1 paper, merged across row chunks):
//   M = max_w M_w,  Z = sum_w Z_w 2^(M_w - M),  S = sum_w acc_w 2^(M_w - M) / Z,
//   lse = (M + log2 Z) * ln 2.
// Prototype axis: the weights are already normalised per row, so the merge is
// the plain ordered sum of the segments' acc.
#include "sa_internal.h"

namespace sa {

// One thread per four consecutive output elements (b, h, j, e..e+3), so the
// partial sums are read as 16-byte vectors; dh is a multiple of 4.  The
// segments of user b are combined in ascending w (the same order for every
// layout, so packed and dense inputs agree bitwise); segments without a
// valid row (M_w = -inf) are skipped.
__global__ __launch_bounds__(256) void sa_merge_kernel(MergeArgs a) {
    const int b = blockIdx.z;
    const int h = blockIdx.y;
    const int q = blockIdx.x * 256 + threadIdx.x;      // quad index within (b, h)
    const int mq = a.m * (a.dh / 4);
    if (q >= mq) return;
    // the quad's (j, e) and the offset of its partial sums within a (slot, h)
    // block of m*dh floats; consecutive threads read consecutive 16 bytes
    int j, e;
    int64_t qoff;
    if (a.lane_major) {
        const int lane = q & 63, blk = q >> 6;         // blk = j16 * (dh/16) + db
        const int db = blk % (a.dh / 16), j16 = blk / (a.dh / 16);
        j = 16 * j16 + (lane & 15);
        e = 16 * db + 4 * (lane >> 4);
        qoff = (int64_t)q * 4;
    } else {
        j = q / (a.dh / 4);
        e = (q - j * (a.dh / 4)) * 4;
        qoff = (int64_t)j * a.dh + e;
    }
    if (offsets_rejected(a.status)) {
        // offsets failed the check: no partial was written; the outputs say so
        const float nan = __builtin_nanf("");
        *(f32x4*)(a.S + (((int64_t)b * a.H + h) * a.m + j) * a.dh + e) = (f32x4){nan, nan, nan, nan};
        if (e == 0 && a.lse) a.lse[((int64_t)b * a.H + h) * a.m + j] = nan;
        return;
    }
    const int64_t total = a.users.total();
    const RowSplit rs = row_split(total, a.G, a.R_fixed, a.R_min, a.split);
    const int64_t us = a.users.vstart(b), ue = a.users.vstart(b + 1);
    const bool empty = ue <= us;
    const int64_t w_first = empty ? 0 : rs.range_of(us);
    const int64_t w_last = empty ? -1 : rs.range_of(ue - 1);
    float* Sb = a.S + (((int64_t)b * a.H + h) * a.m + j) * a.dh + e;
    const int64_t md = (int64_t)a.m * a.dh;

    if (a.norm == 1) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int64_t w = w_first; w <= w_last; ++w)
            acc += *(const f32x4*)(a.part.acc + ((w + b) * a.H + h) * md + qoff);
        *(f32x4*)Sb = acc;
        return;
    }
    // batches of 8 segments: all loads of a batch are issued together (slots
    // past the last segment re-read the last one and are masked), then the
    // running maximum moves once per batch and each segment is scaled once
    const float* Mb = a.part.M + ((int64_t)b * a.H + h) * a.m + j;     // slot w + b = Mb[w * H * m]
    const float* Zb = a.part.Z + ((int64_t)b * a.H + h) * a.m + j;
    const float* Ab = a.part.acc + ((int64_t)b * a.H + h) * md + qoff;
    const int64_t hm = (int64_t)a.H * a.m, hmd = (int64_t)a.H * md;
    float M = -INFINITY, Z = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t w0 = w_first; w0 <= w_last; w0 += 8) {
        float Mw[8], Zw[8];
        f32x4 aw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t w = min(w0 + k, w_last);
            Mw[k] = Mb[w * hm];
            Zw[k] = Zb[w * hm];
            aw[k] = *(const f32x4*)(Ab + w * hmd);
        }
        float bm = M;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (w0 + k <= w_last) bm = fmaxf(bm, Mw[k]);
        // selects, not branches, so that no load is deferred behind the
        // maximum; segments with no valid row add nothing
        const float r = bm > -INFINITY ? exp2f(M - bm) : 1.f;   // 0 while M is -inf
        Z *= r;
        acc *= r;
        M = bm;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool live = w0 + k <= w_last && Mw[k] > -INFINITY;
            const float f = exp2f(Mw[k] - M);
            Z += live ? Zw[k] * f : 0.f;
            const f32x4 t = aw[k] * f;
            acc.x += live ? t.x : 0.f;
            acc.y += live ? t.y : 0.f;
            acc.z += live ? t.z : 0.f;
            acc.w += live ? t.w : 0.f;
        }
    }
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (M > -INFINITY) {
        out = acc / Z;
        lse = (M + log2f(Z)) * kLn2;
    }
    *(f32x4*)Sb = out;
    if (e == 0 && a.lse) a.lse[((int64_t)b * a.H + h) * a.m + j] = lse;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    if (a.users.B == 0) return hipSuccess;
    const int mq = a.m * (a.dh / 4);
    hipLaunchKernelGGL(sa_merge_kernel, dim3((mq + 255) / 256, a.H, a.users.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

// vcu[b] = sum_{b' < b} clamp(lengths[b'], 0, L_max): one block, 1024 threads.
__global__ __launch_bounds__(1024) void sa_dense_vcu_kernel(const int32_t* lengths, int32_t B, int32_t L_max,
                                                             int32_t* vcu) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry = 0;
        vcu[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < B; base += 1024) {
        const int i = base + tid;
        int x = 0;
        if (i < B) {
            x = lengths[i];
            x = x < 0 ? 0 : (x > L_max ? L_max : x);
        }
        // inclusive scan within the wave
        int v = x;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(v, off, 64);
            if (lane >= off) v += y;
        }
        if (lane == 63) wsum[wave] = v;
        __syncthreads();
        int before = carry;
        for (int k = 0; k < wave; ++k) before += wsum[k];
        if (i < B) vcu[i + 1] = before + v;
        __syncthreads();
        if (tid == 1023) carry = before + v;
        __syncthreads();
    }
}

hipError_t launch_dense_vcu(const int32_t* lengths, int32_t B, int32_t L_max, int32_t* vcu, hipStream_t s) {
    hipLaunchKernelGGL(sa_dense_vcu_kernel, dim3(1), dim3(1024), 0, s, lengths, B, L_max, vcu);
    return hipGetLastError();
}

// The debug offsets check: one block walks cu[0..B] (cu == nullptr: dense
// layout, nothing to check), ORs the rule bits of every entry and keeps the
// smallest entry that has any; status[0] = bits, status[1] = that entry or -1.
__global__ __launch_bounds__(256) void sa_check_offsets_kernel(const int32_t* cu, int32_t B, int64_t total_rows,
                                                                int32_t* status) {
    __shared__ int32_t bits_all;
    __shared__ int32_t first;
    if (threadIdx.x == 0) {
        bits_all = 0;
        first = INT32_MAX;
    }
    __syncthreads();
    if (cu) {
        int32_t bits = 0, mine = INT32_MAX;
        for (int32_t b = threadIdx.x; b <= B; b += 256) {
            const int32_t x = offsets_entry_bits(cu, b, B, total_rows);
            bits |= x;
            if (x && b < mine) mine = b;
        }
        if (bits) {
            atomicOr(&bits_all, bits);
            atomicMin(&first, mine);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        status[0] = bits_all;
        status[1] = bits_all ? first : -1;
    }
}

hipError_t launch_check_offsets(const int32_t* cu, int32_t B, int64_t total_rows, int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(sa_check_offsets_kernel, dim3(1), dim3(256), 0, s, cu, B, total_rows, status);
    return hipGetLastError();
}

}  // namespace sa
