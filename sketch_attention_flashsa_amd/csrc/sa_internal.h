// sa_internal.h -- shared definitions of libsketchattn's kernels and host code.
//
// Work decomposition used by every forward kernel (one launch per ragged
// batch, section 4.4 of the SequenceO1 paper):
//   * The valid-length rows of all users, concatenated in user order, form a
//     "virtual row" axis of sigma_L = sum_b L_b positions.  User b occupies
//     [vstart(b), vstart(b+1)).
//   * Row-range block w covers virtual rows [lo(w), lo(w+1)) (RowSplit):
//     R rows each, or -- for the streaming kernel's two blocks per CU --
//     R1 rows for the first G/2 ranges and R2 for the rest.  Its
//     intersection with user b is a "segment"; segment (w, b) stores its
//     partial statistics at slot w + b (distinct for distinct intersecting
//     pairs, at most G + B - 1 slots).
//   * The merge kernel combines the segments of user b in ascending w.
// Because the ranges and the segments depend only on the valid lengths (not
// on the buffer layout), packed and dense+lengths inputs give bitwise-equal
// results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTile = 32;        // rows per streaming tile
constexpr int kRowAlign = 32;    // chunk rows are a multiple of this

// Where user b's rows live and where it sits on the virtual row axis.
struct Users {
    const int32_t* cu;       // packed offsets [B+1] or nullptr (dense)
    const int32_t* vcu;      // dense + lengths: virtual starts [B+1] (workspace)
    int32_t B;
    int32_t L_max;           // dense slot size
    __device__ __forceinline__ int64_t vstart(int b) const {
        if (cu) return (int64_t)cu[b] - cu[0];
        if (vcu) return vcu[b];
        return (int64_t)b * L_max;
    }
    __device__ __forceinline__ int64_t row_base(int b) const {
        return cu ? (int64_t)cu[b] : (int64_t)b * L_max;
    }
    __device__ __forceinline__ int64_t total() const { return vstart(B); }
    // largest b in [0, B) with vstart(b) <= v (v < total())
    __device__ __forceinline__ int find(int64_t v) const {
        int lo = 0, hi = B;  // invariant: vstart(lo) <= v < vstart(hi)
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (vstart(mid) <= v) lo = mid; else hi = mid;
        }
        return lo;
    }
    // find() with its probes spread over the 64 lanes of a wave: one round of
    // independent loads per factor of 64 in B (one round for B <= 64)
    // instead of log2(B) dependent ones, which a kernel otherwise waits for
    // before its first row load.  Lane k of a round probes lo + k (at most 64
    // candidates left) or lo + floor(k (hi - lo) / 64); the largest probe
    // with vstart <= v becomes lo and the next probe hi, so the invariant
    // vstart(lo) <= v < vstart(hi) of find() holds and, for non-decreasing
    // offsets, the result equals find()'s.  Every lane of the wave calls it
    // with the same v.
    __device__ __forceinline__ int find_wave(int64_t v) const {
        const int lane = (int)__lane_id();
        int lo = 0, hi = B;
        while (hi - lo > 1) {
            const int64_t span = hi - lo;
            const int np = span < 64 ? (int)span : 64;            // probes this round
            auto probe = [&](int k) { return span <= 64 ? lo + k : lo + (int)((span * k) >> 6); };
            const bool le = lane < np && vstart(probe(lane)) <= v;
            const uint64_t m = __ballot(le);
            const int k = m ? 63 - __clzll((long long)m) : 0;
            const int nlo = probe(k);
            hi = k + 1 < np ? probe(k + 1) : hi;
            lo = nlo;
        }
        return lo;
    }
};

// Rules of the debug offsets check (SA_FLAG_CHECK_OFFSETS), evaluated for
// entry b of cu[B+1]: bit 1 cu[0] < 0, bit 2 cu[b+1] < cu[b], bit 4
// cu[B] > total_rows.  Host and device run this same code.
constexpr int32_t kOffNegative = 1, kOffDecreasing = 2, kOffPastEnd = 4;
__host__ __device__ __forceinline__ int32_t offsets_entry_bits(const int32_t* cu, int32_t b, int32_t B,
                                                                  int64_t total_rows) {
    int32_t bits = 0;
    if (b == 0 && cu[0] < 0) bits |= kOffNegative;
    if (b < B && cu[b + 1] < cu[b]) bits |= kOffDecreasing;
    if (b == B && (int64_t)cu[B] > total_rows) bits |= kOffPastEnd;
    return bits;
}

// A kernel of a call made with the offsets check runs only when the check
// found nothing: status[0] is the check kernel's verdict (nullptr: no check).
__device__ __forceinline__ bool offsets_rejected(const int32_t* status) {
    return status != nullptr && *status != 0;
}

// Rows per segment: fixed by the caller, or spread evenly over G blocks.
// Row counts are below 2^31 (the entry points check), so the divisions by
// run-time values are 32-bit.
__device__ __forceinline__ int64_t chunk_rows(int64_t total, int G, int R_fixed, int R_min) {
    if (R_fixed > 0) return R_fixed;
    int64_t R = (uint32_t)(total + G - 1) / (uint32_t)G;
    if (R < R_min) R = R_min;
    return (R + kRowAlign - 1) / kRowAlign * kRowAlign;
}

// Row ranges: the first G1 ranges have R1 rows, the others R2 (R1 = R2 = R
// and G1 = G when uniform).  `split` is the share, in percent, of the rows
// that the first half of the ranges takes (50 = uniform).  The streaming
// kernel dispatches the first half of its ranges first; on a CU that holds
// two of its blocks the older one is issued first and runs faster, so a
// split above 50 lets both finish together.  Small inputs, fixed chunk rows
// and splits that would leave a range under R_min rows stay uniform.
struct RowSplit {
    int64_t R1, R2, G1;
    __device__ __forceinline__ int64_t lo(int64_t w) const { return w < G1 ? w * R1 : G1 * R1 + (w - G1) * R2; }
    // the range holding virtual row v (0 <= v < total < 2^31)
    __device__ __forceinline__ int64_t range_of(int64_t v) const {
        return v < G1 * R1 ? (int64_t)((uint32_t)v / (uint32_t)R1)
                           : G1 + (int64_t)((uint32_t)(v - G1 * R1) / (uint32_t)R2);
    }
};
__device__ __forceinline__ RowSplit row_split(int64_t total, int G, int R_fixed, int R_min, int split) {
    const int64_t R = chunk_rows(total, G, R_fixed, R_min);
    const RowSplit uniform = {R, R, (int64_t)G};
    if (R_fixed > 0 || split == 50 || split < 1 || split > 99 || G < 2 || (G & 1)) return uniform;
    const int64_t G1 = G / 2, G2 = G - G1;
    const int64_t even = (uint32_t)(total + G - 1) / (uint32_t)G;     // rows per range if uniform
    const int64_t R1 = (even * split / 50 + kRowAlign - 1) / kRowAlign * kRowAlign;
    if (R1 * G1 >= total) return uniform;
    const int64_t R2 = ((uint32_t)(total - G1 * R1 + G2 - 1) / (uint32_t)G2 + kRowAlign - 1) / kRowAlign * kRowAlign;
    if (R1 < R_min || R2 < R_min) return uniform;
    return {R1, R2, G1};
}

// Partial statistics of the segments.  M and Z are [nslot][H][m].  acc (the
// unnormalised weighted value sums, nslot*H*m*dh floats) has one of two
// layouts, chosen by the kernel that writes it:
//   row-major:  acc[((slot*H + h)*m + j)*dh + e];
//   lane-major: the MFMA accumulator layout, for 16-prototype block j16 and
//     16-wide dh block db, lane l = 16*g + c holds (j = 16*j16 + c,
//     e = 16*db + 4*g + i), i = 0..3, at
//     acc[((((slot*H + h)*(m/16) + j16)*(dh/16) + db)*64 + l)*4 + i],
//     so that each wave stores 1 KB contiguous per accumulator register set.
struct Partials {
    float* acc;
    float* M;     // running maximum, log2 units, scale folded in
    float* Z;     // sum of 2^(x - M)
};

// Address of lane `lane`'s four partial sums of (slot, h, j16, db), lane-major.
__device__ __forceinline__ float* lane_major_acc(const Partials& p, int64_t slot, int H, int h, int m, int dh,
                                                 int j16, int db, int lane) {
    return p.acc + (((((slot * H + h) * (m / 16) + j16) * (dh / 16) + db) * 64 + lane) * 4);
}

struct FwdArgs {
    Users users;
    const uint8_t* mask;     // per buffer row or nullptr
    const void* P;
    int64_t q_batch_stride;  // elements; 0 = shared
    const void* K;
    const void* V;
    int64_t k_stride, v_stride;  // elements between rows
    int32_t H, m, dh;
    float c;                 // scale * log2(e)
    int32_t G;               // row-range blocks
    int32_t R_fixed, R_min;
    int32_t split;           // RowSplit share of the first G/2 ranges (50 = uniform)
    Partials part;
    const float* lse2_tok;   // prototype axis: per (row, head) log2 normaliser
    int32_t norm;            // 0 history, 1 prototype
    const int32_t* status;   // offsets check verdict, or nullptr
    // history axis, streaming kernels: 0 = P * c rounded to bf16 once in the
    // prototype fragments (base-2 products, one rounding of every P element
    // relative to the exact scores); 1 = P enters unrounded and every score
    // is multiplied by c in fp32 (set when the per-prototype lse is requested,
    // whose value keeps the shift that rounding gives the scores)
    int32_t exact_scale;
};

struct MergeArgs {
    Users users;
    int32_t H, m, dh;
    int32_t G, R_fixed, R_min, split;
    Partials part;
    float* S;                // [B][H][m][dh]
    float* lse;              // [B][H][m] or nullptr (history axis only)
    int32_t norm;
    int32_t lane_major;      // acc layout written by the forward kernel
    const int32_t* status;   // offsets check verdict, or nullptr (bad: S, lse = NaN)
};

struct TokLseArgs {
    Users users;
    int64_t total_rows;
    const uint8_t* mask;
    const void* P;
    const void* K;
    int64_t k_stride;
    int32_t H, m, dh;
    float c;
    float* lse2_tok;         // [total_rows][H], log2 units
    float* lse_out;          // [total_rows][H], natural log, or nullptr
    const int32_t* status;   // offsets check verdict, or nullptr (bad: lse_out = NaN)
};

// ---- launchers (return hipGetLastError() of the launch) ----
hipError_t launch_dense_vcu(const int32_t* lengths, int32_t B, int32_t L_max, int32_t* vcu, hipStream_t s);
// status[0] = OR of offsets_entry_bits over b, status[1] = first b with bits (-1: none)
hipError_t launch_check_offsets(const int32_t* cu, int32_t B, int64_t total_rows, int32_t* status, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_f32_forward(const FwdArgs& a, hipStream_t s);
hipError_t launch_f32_tok_lse(const TokLseArgs& a, hipStream_t s);
hipError_t launch_bf16_tok_lse(const TokLseArgs& a, hipStream_t s);

// bf16 MFMA forward: the tile configuration chosen by the host.
struct Bf16Config {
    int protos_per_wave;     // MB: prototypes one wave owns (multiple of 16)
    int waves;               // NW: (head, prototype-block) units per block
    int blocks_per_cu;       // occupancy target used to size G
    int max_heads;           // most heads one block stages
    int k_row, v_row;        // LDS row strides (bytes) of the K and V tiles
    size_t lds_bytes;        // dynamic LDS per block
};
// tile_mb, tile_nw: a requested tile (0, 0 = the default choice)
bool bf16_config(int dh, int m, int H, size_t lds_limit, int tile_mb, int tile_nw, Bf16Config* cfg);
hipError_t launch_bf16_forward(const FwdArgs& a, const Bf16Config& cfg, hipStream_t s);

// bf16 streaming kernel with the direct-to-LDS ring (sa_bf16_stream.hip):
// 8 waves of 32 prototypes per block.
struct StreamConfig {
    int PB;                  // MB-prototype blocks per head
    int MB;                  // prototypes per wave
    int NH;                  // heads per block
    int NW;                  // waves per block
    int groups;              // blocks per row range
    int blocks_per_cu;
};
// prefer_nw: 8 or 16, the block size tried first
bool stream_config(int dh, int m, int H, int prefer_nw, StreamConfig* cfg);
hipError_t launch_bf16_stream(const FwdArgs& a, const StreamConfig& cfg, hipStream_t s);

// Fused key/value projection + forward (sa_fused_proj.hip): X [rows, d_model]
// bf16, W_K / W_V [d_model, H*dh] (W_V == nullptr: V = X), history axis.
struct FusedArgs {
    Users users;             // packed offsets only
    const uint8_t* mask;     // per row or nullptr
    const void* X;
    const void* Wk;
    const void* Wv;          // nullptr: V = X (needs H*dh == d_model)
    const void* P;
    int64_t q_batch_stride;  // elements; 0 = shared
    int32_t H, m, d_model;
    float c;                 // scale * log2(e)
    int32_t G, R_fixed, R_min;
    Partials part;
    const int32_t* status;   // offsets check verdict, or nullptr
};
// One sketch-update launch of stacked refinement (sa_refine.hip).
struct SketchArgs {
    int32_t rows;            // sketch rows: B*m (layer) or m (projection only)
    int32_t m, H, dh;        // D = H*dh features per row
    int32_t mode;            // 0: LN1 + FFN + LN2 [+ queries]; 1: queries only
    const float* base;       // residual input [rows][D], or [m][D] shared (base_shared)
    int32_t base_shared;
    const float* xhat;       // attention output [B][H][m][dh]
    const float* ln1_g;
    const float* ln1_b;
    const float* ln2_g;
    const float* ln2_b;
    const bf16* w1t;         // [2D][D] (W1 transposed)
    const bf16* w3t;         // [2D][D]
    const bf16* w2t;         // [D][2D]
    const bf16* wqt;         // [D][D] next queries' weight transposed, or nullptr
    float eps;
    float* out;              // [rows][D] fp32 (mode 0); may equal base
    bf16* q;                 // [B][H][m][dh] bf16 queries (when wqt)
};
constexpr int kMaxTranspose = 64;
struct TransposeArgs {
    struct Mat {
        const bf16* src;     // [rows][cols]
        bf16* dst;           // [cols][rows]
        int32_t rows, cols;
    } mat[kMaxTranspose];
    int32_t n;
};
// Row projection of the fused entry's two-pass path (sa_refine.hip).
struct ProjectArgs {
    const bf16* X;           // [rows][x_stride]
    int64_t x_stride;
    const bf16* wt;          // [NOUT][DIN] transposed weights
    bf16* out;               // [rows][NOUT]
    int64_t rows;
};
bool project_supported(int din, int nout);
hipError_t launch_project(const ProjectArgs& a, int din, int nout, int grid, hipStream_t s);

bool sketch_supported(int D);
hipError_t launch_sketch(const SketchArgs& a, int D, hipStream_t s);
hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s);

// History-axis backward pass (sa_backward.hip).
constexpr int kBwdTileCols = 256;   // widest K/V row slice (heads x dh) the dP kernel stages
struct BwdArgs {
    Users users;
    const uint8_t* mask;
    const void* P;           // bf16 [H][m][dh] or per user (q_batch_stride)
    int64_t q_batch_stride;
    const void* K;           // bf16 rows
    const void* V;
    int64_t k_stride, v_stride;
    int32_t H, m, dh;
    float c;                 // scale
    float c2;                // scale * log2(e)
    int32_t G;               // row ranges of the dP kernel (and of its partials)
    int32_t G1;              // row ranges of the dK/dV kernel
    int32_t R_fixed, R_min;
    const float* S;          // forward output [B][H][m][dh]
    const float* lse;        // forward lse [B][H][m] (natural log)
    const float* dS;         // upstream gradient [B][H][m][dh]
    float* Dv;               // [B][H][m] dS . S
    float* L2v;              // [B][H][m] lse in log2 units
    bf16* dSb;               // [B][H][m][dh] dS in bf16
    void* dK;                // [rows][H][dh], fp32 or (grads_bf16) bf16
    void* dV;
    int32_t grads_bf16;
    Partials part;           // dP partials (acc only, lane-major)
    float* dP;               // [H][m][dh] or [B][H][m][dh]
    int32_t per_user;
    int32_t dp_register_staged;  // 1: the register-staged dP kernel for every shape
};
bool bwd_supported(int dh, int m);
void bwd_dp_shape(int m, int H, int* NH, int* PB);
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);

// STCA single-query attention, reordered (sa_stca.hip).
constexpr int kStcaTargets = 16;     // targets per block (one MFMA column tile)
struct StcaArgs {
    const bf16* X;           // history rows, x_stride elements apart
    int64_t x_stride;
    const bf16* qm;          // [T][D] queries x W_Q (bf16)
    const bf16* wk;          // [D][D] W_K as given ([in][out])
    const int32_t* cu;       // [B+1] rows of each user
    const int32_t* tcu;      // [B+1] targets of each user
    const int32_t* win;      // [T][2] per-target row window, or nullptr
    bf16* y;                 // [T][h][D] out: alpha X per target and head
    int4* table;             // [grid][2] per block: (user, first target, targets, head pair) and
                             // (first row of the rows its targets see, their count, 0, 0); user -1 = idle
    int32_t B, T, h, D, grid;
    float c;                 // score scale * log2(e)
};
bool stca_supported(int D, int dh);
hipError_t launch_stca(const StcaArgs& a, int dh, hipStream_t s);

// Batched bf16 GEMM, both operands k-contiguous (sa_gemm.hip):
// C[z][m][n] = sum_k A[z][m][k] Bt[z][n][k]; K a multiple of 32, N of 4,
// lda and ldb multiples of 8, ldc of 4; C bf16 or fp32.
struct GemmArgs {
    const bf16* A;
    const bf16* Bt;
    void* C;
    int64_t lda, ldb, ldc, sA, sB, sC;
    int32_t M, N, K, batch;
};
hipError_t launch_gemm_nt(const GemmArgs& a, bool out_bf16, hipStream_t s);

bool fused_supported(int d_model, int m, int dh);
int fused_groups(int H);     // blocks per row range
hipError_t launch_fused(const FusedArgs& a, hipStream_t s);

}  // namespace sa
