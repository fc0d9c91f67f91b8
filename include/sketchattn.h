/*
 * sketchattn.h -- C ABI of libsketchattn, Sketch Attention (SA) on AMD
 * Instinct MI355X (gfx950).
 *
 * SA (SequenceO1 paper, section 3.1 "Sketch Attention (SA)" and appendix A.4)
 * compresses one user's history of n behaviour rows into a fixed-size sketch
 * of m rows ("prototypes", the paper's k):
 *
 *     score   s[j,i]     = scale * < P[h,j,:], K[i,h,:] >
 *     weight  A[j,i]     = softmax of s over one axis (see sa_norm)
 *     sketch  S[b,h,j,:] = sum_i A[j,i] * V[i,h,:]
 *
 * for every user b and head h.  The library computes it the way section 4.4
 * (FlashSA) describes: score blocks, running softmax statistics (maximum and
 * log-sum-exp) and the weighted aggregation are fused and streamed, so the
 * m x n score matrix never reaches device memory, and a whole ragged batch of
 * users is served by one pass.
 *
 * Conventions for every entry point below
 *   - All data pointers are DEVICE memory owned by the caller; the library
 *     never allocates, frees or retains them.  Inputs are read-only; outputs
 *     are fully overwritten.
 *   - Work is enqueued asynchronously on `stream`; no call synchronises with
 *     the device or reads device memory from the host (offsets, lengths and
 *     masks stay on the device).
 *   - Results are deterministic: the same call on the same device gives
 *     bitwise-identical outputs (fixed reduction order, no float atomics).
 *     The row segmentation depends only on the problem and the device's CU
 *     count (and on sa_set_tuning(), which nothing calls unless a caller
 *     asks for a non-default work split); the environment plays no part.
 *   - Errors that the host can detect (null or misaligned pointers, bad
 *     sizes, unsupported shapes, a short workspace) return a non-zero status
 *     before anything is enqueued; sa_last_error() then describes it.  No C++
 *     exception crosses this interface.  Offsets live in device memory and
 *     are trusted by default: they must satisfy the stated rules or results
 *     are undefined.  SA_FLAG_CHECK_OFFSETS (below) makes the forward entry
 *     points validate them on the device first.
 *   - Thread safety: calls may be made from several host threads; the only
 *     per-thread state is the error text, the timing events and the tuning
 *     below.
 */
#ifndef SKETCHATTN_H
#define SKETCHATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_VERSION_MAJOR 0
#define SA_VERSION_MINOR 1
#define SA_VERSION_PATCH 0

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, negative or inconsistent size */
    SA_ERR_UNSUPPORTED = 2,  /* valid request outside the compiled shapes (see sa_forward) */
    SA_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than the query says */
    SA_ERR_HIP = 4           /* the HIP runtime reported an error when launching */
} sa_status;

/* Element type of P, K, V (and X, Wk, Wv). */
typedef enum sa_dtype {
    SA_DTYPE_F32 = 0,  /* IEEE binary32; no rounding to a narrower type anywhere */
    SA_DTYPE_BF16 = 1  /* bfloat16 storage; products accumulate in fp32 */
} sa_dtype;

/*
 * Which axis the softmax normalises.
 *   SA_NORM_HISTORY   (default) one distribution per prototype over the
 *                     user's valid rows: sum_i A[j,i] = 1.  With P = 0 the
 *                     sketch is the mean of V.  This is the prototype-query
 *                     attention S = softmax_L(P_h K_b^T * scale) V_b.
 *   SA_NORM_PROTOTYPE one distribution per row over the m prototypes:
 *                     sum_j A[j,i] = 1 -- the normalisation display of the
 *                     paper's section 3.1 -- with the sketch X~ = A V taken
 *                     as written (no renormalisation over rows).
 */
typedef enum sa_norm {
    SA_NORM_HISTORY = 0,
    SA_NORM_PROTOTYPE = 1
} sa_norm;

typedef struct sa_problem {
    int32_t B;              /* users (>= 0) */
    int32_t H;              /* heads (>= 1) */
    int32_t m;              /* prototypes per head (>= 1) */
    int32_t dh;             /* width of one head (>= 1) */
    int64_t total_rows;     /* rows of the K/V (or X) buffers; packed: >= cu_offsets[B];
                               dense: 0 or >= B * L_max */
    int32_t L_max;          /* dense layout: row slots per user; must be 0 for packed */
    int32_t dtype;          /* sa_dtype */
    int32_t norm;           /* sa_norm */
    float scale;            /* score scale; 0 means 1/sqrt(dh) */
    int64_t k_row_stride;   /* elements between consecutive rows of K; 0 means H*dh */
    int64_t v_row_stride;   /* elements between consecutive rows of V; 0 means H*dh */
    int64_t q_batch_stride; /* elements between users' prototype sets in P; 0 means one
                               shared set P[H, m, dh] (the paper shares prototypes
                               across users, section 3.1) */
    int32_t chunk_rows;     /* 0: automatic work split over the device; > 0: every work
                               segment covers this many rows (multiple of 32) */
    int32_t flags;          /* OR of the SA_FLAG_* bits below that the entry point
                               accepts; 0 for the default behaviour */
} sa_problem;

/* sa_problem.flags bit for sa_backward only: dK and dV are written as bf16
 * (the fp32 sums rounded to nearest even), the element type of K and V. */
#define SA_FLAG_BF16_GRADS 1

/*
 * sa_problem.flags bit for sa_forward and sa_forward_fused_proj (a debug
 * aid): before any kernel reads an offset, a small kernel checks cu_offsets
 * on the device against the rules of sa_forward (the batching of ragged user
 * histories that section 4.4 of the SequenceO1 paper serves in one pass):
 *     rule 1 (bit 1)  cu_offsets[0] >= 0
 *     rule 2 (bit 2)  cu_offsets[b] <= cu_offsets[b+1] for every b
 *     rule 3 (bit 4)  cu_offsets[B] <= total_rows
 * and writes the result into the first 8 bytes of the workspace: int32
 * status (0 = valid, else the OR of the violated rules' bits) and int32
 * index (the smallest b at which a rule fails: 0 for rule 1, the b of the
 * first decreasing pair for rule 2, B for rule 3; -1 when valid).  Every
 * later kernel of the call reads the status first; when it is non-zero none
 * of them reads K, V, X or the mask, and S_out and lse_out are filled with
 * NaN.  The host never reads the status on the call path (the call stays
 * asynchronous): read it from the workspace after synchronising.  The
 * dense layout (cu_offsets == NULL) has nothing to check (lengths are
 * clamped) and always gets status 0.  The flag adds 256 bytes to the
 * workspace size; the rest of the workspace follows the status section.
 */
#define SA_FLAG_CHECK_OFFSETS 2

/*
 * The rules of SA_FLAG_CHECK_OFFSETS evaluated on the host, for offsets the
 * caller holds in host memory (the device check runs the same rule code).
 * cu_offsets_host has B+1 entries.  Returns the status word described above
 * and stores the index of the first violation in *first_bad (if non-NULL).
 */
int32_t sa_check_offsets_host(const int32_t* cu_offsets_host, int32_t B, int64_t total_rows, int32_t* first_bad);

/*
 * Sketch Attention forward over a ragged batch of user histories.
 *
 * Operation: SequenceO1 paper, section 3.1 (scores, normalisation, sketch
 * construction) and appendix A.4; fused and streamed as in section 4.4.
 *
 * P           [H, m, dh] (or [B, ...] via q_batch_stride), dtype.  Head h uses
 *             P[h]; head h of a row is its channels [h*dh, (h+1)*dh).
 * K, V        packed: [total_rows, H, dh] rows, user b owning rows
 *             [cu_offsets[b], cu_offsets[b+1]);
 *             dense (cu_offsets == NULL): [B, L_max, H, dh], user b owning
 *             rows b*L_max + [0, len_b), len_b = min(lengths[b], L_max), or
 *             L_max when lengths == NULL.  dh is contiguous and the H heads
 *             of a row are contiguous; rows are k_row_stride / v_row_stride
 *             elements apart.  bf16 rows must start on 16-byte boundaries.
 * cu_offsets  int32 [B+1], non-decreasing, cu_offsets[0] >= 0,
 *             cu_offsets[B] <= total_rows; rows outside every user are never
 *             read.  NULL selects the dense layout.
 * lengths     int32 [B] (dense only, optional); negative counts as 0.
 * mask        uint8, one byte per row of the K/V buffers (dense: [B, L_max]),
 *             optional; 0 excludes the row (it is never read as a number, so
 *             NaN or Inf there cannot leak).  A user with no valid row is
 *             empty.
 * S_out       float32 [B, H, m, dh], 16-byte aligned.  Empty users get 0.
 * lse_out     optional float32.  HISTORY: [B, H, m], natural-log
 *             log-sum-exp of the scaled scores over the user's valid rows
 *             (-inf for empty users).  PROTOTYPE: [total_rows, H], the
 *             log-sum-exp over the m prototypes of each row (-inf for rows
 *             that are masked or belong to no user).  Requesting it makes
 *             the bf16 kernels apply the scale to unrounded score products
 *             (without it they may fold the scale into the prototypes,
 *             rounded once to bf16, which shifts a normaliser by about 2^-9
 *             of the scores but cancels in S); S from the two agrees within
 *             the bf16 tolerance, not bitwise.
 * workspace   device scratch of at least sa_forward_workspace_size(pb)
 *             bytes, 256-byte aligned; contents need no initialisation and
 *             are clobbered.  May be NULL when the query returns 0.
 * stream      HIP stream the work is enqueued on.
 *
 * Compiled shapes: bf16: dh in {32, 64, 128}, m a multiple of 16 (the
 * direct-to-LDS streaming kernel for dh in {32, 64} with m a multiple of 32,
 * and for dh == 128 with m a multiple of 256; a register-staged kernel for
 * the rest).
 * f32: dh in {16, 32, 64, 128}, any m.  The prototype axis takes shared
 * prototypes only (q_batch_stride == 0).  Others return SA_ERR_UNSUPPORTED.
 */
sa_status sa_forward(const sa_problem* pb, const void* P, const void* K, const void* V,
                     const int32_t* cu_offsets, const int32_t* lengths, const uint8_t* mask,
                     float* S_out, float* lse_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Bytes of workspace sa_forward needs for this problem on the current device
 * (0 if the problem itself is invalid; sa_last_error() then says why). */
size_t sa_forward_workspace_size(const sa_problem* pb);

/*
 * sa_forward without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * kernels, results (bitwise) and errors as sa_forward, minus workspace and
 * workspace_bytes: the workspace is an array of
 * sa_forward_noalloc_max_workspace() bytes (64 MiB) that the library holds
 * on each device it runs on, from the first call on that device until the
 * process ends.  A problem whose sa_forward_workspace_size() exceeds it
 * returns SA_ERR_WORKSPACE before anything is enqueued (the 100K-row
 * workload of the benchmark needs about 39 MB on the history axis).
 * The array is shared by every call on a device and keeps the last call's
 * contents: calls that overlap on one device (different streams or threads
 * without ordering between them) race on it, so order them on one stream or
 * use sa_forward.  Nothing in it needs to start zeroed.  With
 * SA_FLAG_CHECK_OFFSETS the status words are the first 8 bytes of that
 * array, which the caller cannot read: use sa_forward to inspect them (S_out
 * and lse_out still come back NaN on bad offsets).
 */
sa_status sa_forward_noalloc(const sa_problem* pb, const void* P, const void* K, const void* V,
                             const int32_t* cu_offsets, const int32_t* lengths, const uint8_t* mask, float* S_out,
                             float* lse_out, hipStream_t stream);

/* Bytes of the per-device workspace array of sa_forward_noalloc. */
size_t sa_forward_noalloc_max_workspace(void);

/* Name of the kernel that performs the pass over K/V for this problem on the
 * current device (the one the timing events below bracket): a static string,
 * or NULL if the problem is invalid or unsupported (sa_last_error() says why).
 * Profilers use it to find that kernel in a trace. */
const char* sa_forward_kernel_name(const sa_problem* pb);

/*
 * Fused key/value projection + Sketch Attention forward (packed layout only).
 *
 * Operation: the key projection K = X W_K of the paper's section 3.1 scores
 * (costed in appendix G.3), and V = X W_V, computed on chip tile by tile and
 * consumed at once by the sa_forward computation above, so K and V never
 * reach device memory.  K and V are rounded to bf16 before the score and
 * aggregation products (fp32 accumulation throughout).
 *
 * X        [total_rows, d_model], dtype (bf16 only), rows 16-byte aligned.
 * Wk, Wv   [d_model, H*dh] row-major: K[i, h*dh + e] = sum_c X[i,c] Wk[c, h*dh + e].
 *          Wv == NULL means V = X (the paper's sketch aggregates X itself,
 *          section 3.1); that requires H*dh == d_model.
 * P, cu_offsets, mask, S_out, lse_out, workspace, stream: as for sa_forward
 *          (pb->L_max must be 0, pb->k_row_stride and v_row_stride are ignored).
 *
 * Compiled shapes: bf16, history axis (SA_NORM_HISTORY), dh == 32,
 * d_model in {128, 256}, m in {64, 128, 256}; P shared or per user
 * (q_batch_stride); any H.  Two-pass shapes: Wv == NULL (V = X) with
 * H*dh == d_model in {128, 256}, shared P and a (dh, m, H) that sa_forward
 * streams (for example the paper's single head of width 128 with m = 1024,
 * appendix G.5): K = X Wk is first projected into the workspace (bf16), then
 * the sa_forward pass runs on it, so K makes one round trip through memory.
 * Others return SA_ERR_UNSUPPORTED.  S_out is 16-byte aligned; X, Wk, Wv and
 * P are 16-byte aligned.
 */
sa_status sa_forward_fused_proj(const sa_problem* pb, const void* X, int32_t d_model,
                                const void* Wk, const void* Wv, const void* P,
                                const int32_t* cu_offsets, const uint8_t* mask,
                                float* S_out, float* lse_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace sa_forward_fused_proj needs on the current device. */
size_t sa_forward_fused_proj_workspace_size(const sa_problem* pb, int32_t d_model);

/*
 * Backward pass of sa_forward, history axis (the paper trains SA end to end;
 * the gradient is the chain rule through section 3.1's weighted sum and the
 * softmax over each user's rows).  With A_ji = exp(c P_j.K_i - lse_j) over
 * user b's valid rows i, and dS the gradient arriving at S:
 *     dV_i = sum_j A_ji dS_j
 *     ds_ji = A_ji (dS_j.V_i - dS_j.S_j)
 *     dK_i = c sum_j ds_ji P_j,      dP_j = c sum_i ds_ji K_i
 * (dP summed over users when P is shared).  The weights are recomputed from
 * the forward's saved lse; P, K, V and dS enter the MFMA products in bf16,
 * everything accumulates in fp32.
 *
 * pb, P, K, V, cu_offsets, lengths, mask: exactly as given to sa_forward.
 * S, lse   the forward's outputs [B, H, m, dh] and [B, H, m] (lse is required).
 * dS       [B, H, m, dh] fp32 upstream gradient.
 * dP       fp32, shaped like P ([H, m, dh], or [B, H, m, dh] with per-user P).
 * dK, dV   [rows, H, dh] (packed) or [B, L_max, H, dh] (dense), dh
 *          contiguous, heads contiguous in a row, 16-byte aligned; fp32, or
 *          bf16 when pb->flags has SA_FLAG_BF16_GRADS.  Every row of a user
 *          (valid or masked) is written; masked rows get 0.  Rows outside
 *          every user and dense padding past L_b are left as they are.
 * workspace, workspace_bytes: at least sa_backward_workspace_size(pb).
 *
 * Compiled shapes: bf16, history axis, dh in {32, 64}, m in {32, 64, 128,
 * 256}; any H; P shared or per user.  Others return SA_ERR_UNSUPPORTED.
 * P, K, V, S, dS, dP, dK and dV are 16-byte aligned.  Deterministic: dP's partial
 * sums are added in a fixed order, no float atomics.
 */
sa_status sa_backward(const sa_problem* pb, const void* P, const void* K, const void* V,
                      const int32_t* cu_offsets, const int32_t* lengths, const uint8_t* mask,
                      const float* S, const float* lse, const float* dS, float* dP, void* dK,
                      void* dV, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace sa_backward needs on the current device (0 if the
 * problem is invalid or unsupported; sa_last_error() says why).  pb->L_max
 * > 0 means the dense layout, else packed. */
size_t sa_backward_workspace_size(const sa_problem* pb);

/*
 * Stacked Sketch Attention refinement (section 3.3 of the SequenceO1 paper),
 * n_layers layers over a packed ragged batch.  The sketch starts as the
 * prototypes, Xt_0 = P0 [m, d]; layer l computes, for every user b,
 *     Q    = Xt_l Wq_l                      (queries from the current sketch)
 *     Xhat = softmax_L(Q (X_b Wk_l)^T / sqrt(dh)) X_b   per head (values = X)
 *     Xbar = LN(Xt_l + Xhat; ln1_g, ln1_b)
 *     Xt_{l+1} = LN(Xbar + (silu(Xbar W1) * (Xbar W3)) W2; ln2_g, ln2_b)
 * where head h uses channels [h*dh, (h+1)*dh) of Q, K and X, LN is a per-row
 * layer norm over the d channels with eps inside the square root, and the
 * FFN is SwiGLU with inner width 2d (appendix G of the paper) and no biases.
 * The attention pass of each layer is sa_forward_fused_proj's (keys
 * projected on chip, never written to memory); the sketch update runs on
 * MFMA with fp32 layer norms.  Queries, keys and the FFN's inputs and hidden
 * units are rounded to bf16 before their products (fp32 accumulation).
 *
 * pb       B, H, m, dh (d = H*dh = d_model), total_rows, dtype BF16, norm
 *          SA_NORM_HISTORY, scale (0: 1/sqrt(dh)); q_batch_stride, L_max and
 *          the row strides must be 0.
 * X        [total_rows, d_model] bf16 history rows (the values), packed by
 *          cu_offsets [B+1] as in sa_forward; mask optional per row.
 * P0       [m, d_model] fp32 prototypes.
 * layers   host array of n_layers (1..8) descriptors; every pointer in them is
 *          device memory: Wq, Wk [d, d] and W1, W3 [d, 2d] and W2 [2d, d],
 *          bf16, row-major [in, out] (y = x W); ln*_g, ln*_b [d] fp32.
 * eps      layer-norm epsilon (> 0 recommended; 1e-5 is the usual value).
 * out      [B, m, d_model] fp32: the final sketch Xt_{n_layers}.
 * workspace, workspace_bytes: at least sa_refine_workspace_size(pb, d_model,
 *          n_layers) bytes, 256-byte aligned, owned by the caller.
 *
 * Compiled shapes: dh == 32, d_model in {128, 256}, m in {64, 128, 256}.
 * Others return SA_ERR_UNSUPPORTED.  X, P0, out and every matrix are 16-byte
 * aligned.  Users with no valid row get Xhat = 0.
 */
typedef struct sa_refine_layer {
    const void* Wq;
    const void* Wk;
    const float* ln1_g;
    const float* ln1_b;
    const void* W1;
    const void* W3;
    const void* W2;
    const float* ln2_g;
    const float* ln2_b;
} sa_refine_layer;

sa_status sa_refine_forward(const sa_problem* pb, const void* X, int32_t d_model, const float* P0,
                            int32_t n_layers, const sa_refine_layer* layers, float eps,
                            const int32_t* cu_offsets, const uint8_t* mask, float* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace sa_refine_forward needs on the current device (0 if the
 * problem is invalid; sa_last_error() says why). */
size_t sa_refine_workspace_size(const sa_problem* pb, int32_t d_model, int32_t n_layers);

/*
 * STCA single-query target-to-history cross attention, reordered.
 *
 * Operation: section 2.3 of the SequenceO1 paper ("STCA Recap") defines the
 * attention of one target vector x over a history X [L, D] with h heads of
 * width dh = D / h as softmax((x W_Q)(X W_K)^T / sqrt(dh)) (X W_V); appendix
 * G.2.1 evaluates it without the L x dh key and value projections.  Per head
 * (channels c = [hh*dh, (hh+1)*dh) of the projections):
 *     u      = (x W_Q[:, c]) W_K[:, c]^T          [D]
 *     alpha  = softmax(scale * u X^T)             over the target's rows
 *     out[c] = (alpha X) W_V[:, c]                [dh]
 * This entry does that for every target of a packed ragged batch: q = x W_Q
 * for all targets (one GEMM), then one fused attention kernel that forms u,
 * the weights and alpha X on chip, then the per-head products with W_V (one
 * batched GEMM); plus a weight transpose and a small setup launch.  The
 * targets of one user share the user's rows (the multi-request batching of
 * section 4.2), so each pass over a user's rows serves 16 of its targets for
 * two heads.  The products run on MFMA in bf16 with fp32 accumulation; q and
 * u, the weights and alpha X are rounded to bf16 before their products.  The
 * output projection W_O and the query-side FFN of a full STCA layer are
 * one-token transforms outside this entry.
 *
 * pb        B users, T targets, width D, heads h, total_rows of X,
 *           x_row_stride (elements between rows of X; 0 means D), scale (0:
 *           1/sqrt(dh)), flags (must be 0).
 * xt        [T, D] bf16 target vectors.
 * X         [total_rows, D] bf16 history rows (x_row_stride apart); user b
 *           owns rows [cu_offsets[b], cu_offsets[b+1]).  Rows of a user must
 *           be finite (a row outside one target's window still meets the
 *           others' weights).
 * Wq, Wk, Wv [D, D] bf16 row-major, [in, out]: q = x Wq.
 * cu_offsets int32 [B+1], non-decreasing, cu_offsets[B] <= total_rows.
 * t_offsets  int32 [B+1], non-decreasing, t_offsets[B] <= T: the targets of
 *           user b are t_offsets[b] .. t_offsets[b+1]-1.  Targets outside
 *           every user get out = 0.
 * windows   int32 [T, 2] or NULL: target t sees only rows [lo, hi) of its
 *           user (relative to the user's first row, clipped to the user): the
 *           request-aware masking of section 4.2.  An empty window gives 0.
 * out       [T, D] fp32: the h head outputs side by side.
 * workspace at least sa_stca_workspace_size(pb) bytes, 256-byte aligned.
 *
 * Compiled shapes: D == 1024 with h in {16, 8} (dh 64 or 128; the paper's
 * STCA uses h = 16, appendix G.5).  Others return SA_ERR_UNSUPPORTED.  xt,
 * X, the matrices and out are 16-byte aligned.  Deterministic.
 */
typedef struct sa_stca_problem {
    int32_t B;              /* users (>= 0) */
    int32_t T;              /* targets (>= 0) */
    int32_t D;              /* model width */
    int32_t h;              /* heads; dh = D / h */
    int64_t total_rows;     /* rows of X */
    int64_t x_row_stride;   /* elements between rows of X; 0 means D */
    float scale;            /* score scale; 0 means 1/sqrt(dh) */
    int32_t flags;          /* reserved, must be 0 */
} sa_stca_problem;

sa_status sa_stca_attention(const sa_stca_problem* pb, const void* xt, const void* X, const void* Wq,
                            const void* Wk, const void* Wv, const int32_t* cu_offsets,
                            const int32_t* t_offsets, const int32_t* windows, float* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace sa_stca_attention needs (0 if the problem is invalid or
 * unsupported; sa_last_error() says why). */
size_t sa_stca_workspace_size(const sa_stca_problem* pb);

/*
 * Work-split tuning for sweeps and benchmarks (not part of the computation).
 * Each field left 0 keeps the library's default, which is what every call
 * uses unless this is called.  The settings change which rows a work segment
 * covers, and so the order in which sums are rounded: results move within
 * the stated tolerances and stay bitwise repeatable for fixed settings.
 * Thread-local: they apply to the calls this host thread makes until the next
 * sa_set_tuning(); NULL restores the defaults.  Invalid values return
 * SA_ERR_INVALID_ARG and leave the settings unchanged.
 */
typedef struct sa_tuning {
    int32_t register_staged;   /* 1: bf16 forward on the register-staged kernel
                                  instead of the direct-to-LDS streaming kernel */
    int32_t stream_waves;      /* 8 or 16: preferred streaming block size */
    int32_t blocks_per_cu;     /* > 0: occupancy that sizes the forward's row split */
    int32_t range_split;       /* 1..99: percent of the rows that the first half of
                                  the streaming kernel's row ranges takes when two
                                  blocks share a CU (50 = equal ranges) */
    int32_t bf16_tile_mb;      /* register-staged kernel: prototypes per wave (16, 32, 64) */
    int32_t bf16_tile_nw;      /* register-staged kernel: waves per block (4, 8) */
    int32_t bwd_blocks_per_cu; /* > 0: occupancy that sizes the backward's dK/dV row split */
    int32_t bwd_dp_register_staged; /* 1: backward dP pass on the register-staged kernel */
} sa_tuning;

sa_status sa_set_tuning(const sa_tuning* tuning);

/*
 * Timing hook for benchmarks and profilers (not part of the computation).
 * When both events are non-NULL, the next sa_forward or sa_forward_fused_proj
 * call made on this host thread records `start` on its stream immediately
 * before the streaming kernel (the pass over K/V or X; on the fused entry's
 * two-pass shapes, before the key projection) and `stop` immediately after
 * it, then forgets both; the next sa_refine_forward or sa_backward call
 * records them before its first and after its last launch; the next
 * sa_stca_attention call records them around its launches after the weight
 * transpose (query GEMM, attention, output GEMM).
 * NULL, NULL clears a pending request, and so does the next call of any
 * entry point above, including one that fails before launching anything.
 * The events belong to the caller (hipEventCreate); the library never
 * creates, waits on or destroys them.  Returns SA_ERR_INVALID_ARG if exactly
 * one is NULL.
 */
sa_status sa_set_timing_events(hipEvent_t start, hipEvent_t stop);

/* Static text for a status code.  Takes any integer (a code read back from a
 * log or another language need not be one of the sa_status values): codes
 * outside sa_status give "unknown status".  Never NULL; the text is static. */
const char* sa_status_string(int32_t status);

/* Detail of the last failing call on this host thread ("" if none). */
const char* sa_last_error(void);

/* SA_VERSION_MAJOR * 10000 + SA_VERSION_MINOR * 100 + SA_VERSION_PATCH. */
int sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKETCHATTN_H */
