/*
 * sa_oracle.c -- plain, slow, double-precision CPU reference for Sketch Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no header, helper or constant with the GPU
 * library: the problem description below is its own.
 *
 * What it computes (SequenceO1 paper, section 3.1 "Sketch Attention (SA)" and
 * appendix A.4 "Sketch Attention as an Implicit Length Projection"):
 *   scores   s[j,i] = scale * <P[h,j,:], K[i,h,:]>           (prototype j, token i)
 *   HISTORY   axis: A[j,i] = exp(s[j,i]) / sum_i' exp(s[j,i'])  (softmax over the
 *                   user's valid history rows, one distribution per prototype)
 *   PROTOTYPE axis: A[j,i] = exp(s[j,i]) / sum_j' exp(s[j',i])  (softmax over the
 *                   m prototypes, one distribution per token, so that
 *                   sum_j A[j,i] = 1: the normalisation display of section 3.1)
 *   sketch   S[b,h,j,:] = sum_i A[j,i] * V[i,h,:]              (X~ = A X)
 * The history-axis reading is the default; both axes are provided.
 *
 * Method: for every (user, head, prototype) the scores are computed in double
 * from inputs widened exactly from their stored type; then a first pass takes
 * the maximum, a second pass sums exp(s - max) in ascending row order and
 * accumulates the weighted values.  No online rescaling, no blocking.
 *
 * Layouts: K and V are [rows, H, dh] with per-row strides (elements).  Either
 * packed (cu != NULL: user b owns rows [cu[b], cu[b+1])) or dense (cu == NULL:
 * user b owns rows [b*L_max, b*L_max + len_b), len_b = lengths[b] or L_max).
 * mask (optional, per row): 0 excludes the row from every sum and max.
 * An empty user (no valid rows) yields S = 0 and lse = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SAO_F32 0
#define SAO_BF16 1
#define SAO_F64 2

#define SAO_HISTORY 0
#define SAO_PROTOTYPE 1

typedef struct {
    int32_t B, H, m, dh;
    int64_t total_rows;
    int32_t L_max;        /* dense layout when cu == NULL */
    int32_t in_dtype;     /* SAO_F32 / SAO_BF16 / SAO_F64 */
    int32_t norm;         /* SAO_HISTORY / SAO_PROTOTYPE */
    double scale;         /* <= 0 means 1/sqrt(dh) */
    int64_t k_row_stride; /* elements; 0 means H*dh */
    int64_t v_row_stride; /* elements; 0 means H*dh */
    int64_t p_user_stride;/* elements between users' prototype sets; 0 = shared */
} sao_problem;

/* ---- exact widening of one stored element to double ---- */
static double widen(const void* base, int dtype, int64_t idx) {
    if (dtype == SAO_F32) return (double)((const float*)base)[idx];
    if (dtype == SAO_F64) return ((const double*)base)[idx];
    /* bf16: the upper 16 bits of an IEEE binary32 */
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double scale_of(const sao_problem* pb) {
    return pb->scale > 0 ? pb->scale : 1.0 / sqrt((double)pb->dh);
}
static int64_t kstride(const sao_problem* pb) { return pb->k_row_stride ? pb->k_row_stride : (int64_t)pb->H * pb->dh; }
static int64_t vstride(const sao_problem* pb) { return pb->v_row_stride ? pb->v_row_stride : (int64_t)pb->H * pb->dh; }

/* rows owned by user b, before masking */
static void user_rows(const sao_problem* pb, const int32_t* cu, const int32_t* lengths, int b,
                      int64_t* first, int64_t* count) {
    if (cu) {
        *first = cu[b];
        *count = (int64_t)cu[b + 1] - cu[b];
    } else {
        int64_t len = lengths ? lengths[b] : pb->L_max;
        if (len > pb->L_max) len = pb->L_max;
        if (len < 0) len = 0;
        *first = (int64_t)b * pb->L_max;
        *count = len;
    }
}

/* Collect the valid rows of user b (mask applied) into a fresh array. */
static int64_t valid_rows(const sao_problem* pb, const int32_t* cu, const int32_t* lengths,
                          const uint8_t* mask, int b, int64_t** out) {
    int64_t first, count;
    user_rows(pb, cu, lengths, b, &first, &count);
    int64_t* r = (int64_t*)malloc(sizeof(int64_t) * (size_t)(count > 0 ? count : 1));
    int64_t n = 0;
    for (int64_t i = 0; i < count; ++i) {
        int64_t row = first + i;
        if (mask && mask[row] == 0) continue;
        r[n++] = row;
    }
    *out = r;
    return n;
}

/* score of prototype j of head h against row `row`, scale included */
static double score(const sao_problem* pb, const void* P, const void* K, int b, int h, int j, int64_t row) {
    const int64_t pbase = (int64_t)b * pb->p_user_stride + ((int64_t)h * pb->m + j) * pb->dh;
    const int64_t kbase = row * kstride(pb) + (int64_t)h * pb->dh;
    double acc = 0.0;
    for (int e = 0; e < pb->dh; ++e)
        acc += widen(P, pb->in_dtype, pbase + e) * widen(K, pb->in_dtype, kbase + e);
    return acc * scale_of(pb);
}

/* History axis, one (b, h, j): out[dh] and *lse.  s is scratch of n doubles. */
static void history_one(const sao_problem* pb, const void* P, const void* K, const void* V,
                        const int64_t* rows, int64_t n, int b, int h, int j, double* s,
                        double* out, double* lse) {
    for (int e = 0; e < pb->dh; ++e) out[e] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double M = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {          /* pass 1: scores and their maximum */
        s[t] = score(pb, P, K, b, h, j, rows[t]);
        if (s[t] > M) M = s[t];
    }
    double Z = 0.0;
    for (int64_t t = 0; t < n; ++t) {          /* pass 2: weights, sum, weighted values */
        const double w = exp(s[t] - M);
        Z += w;
        const int64_t vbase = rows[t] * vstride(pb) + (int64_t)h * pb->dh;
        for (int e = 0; e < pb->dh; ++e) out[e] += w * widen(V, pb->in_dtype, vbase + e);
    }
    for (int e = 0; e < pb->dh; ++e) out[e] /= Z;
    *lse = M + log(Z);
}

/* Prototype axis, one (b, h): all m rows of S[b,h] and lse_tok[row, h]. */
static void prototype_bh(const sao_problem* pb, const void* P, const void* K, const void* V,
                         const int64_t* rows, int64_t n, int b, int h, double* S_bh, double* lse_tok) {
    const int m = pb->m, dh = pb->dh;
    double* s = (double*)malloc(sizeof(double) * (size_t)m);
    for (int64_t x = 0; x < (int64_t)m * dh; ++x) S_bh[x] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const int64_t row = rows[t];
        double M = -INFINITY;
        for (int j = 0; j < m; ++j) {          /* pass 1 over prototypes */
            s[j] = score(pb, P, K, b, h, j, row);
            if (s[j] > M) M = s[j];
        }
        double Z = 0.0;
        for (int j = 0; j < m; ++j) Z += exp(s[j] - M);   /* pass 2 */
        const int64_t vbase = row * vstride(pb) + (int64_t)h * dh;
        for (int j = 0; j < m; ++j) {
            const double a = exp(s[j] - M) / Z;
            for (int e = 0; e < dh; ++e) S_bh[(int64_t)j * dh + e] += a * widen(V, pb->in_dtype, vbase + e);
        }
        if (lse_tok) lse_tok[row * pb->H + h] = M + log(Z);
    }
    free(s);
}

static int check(const sao_problem* pb) {
    if (!pb || pb->B < 0 || pb->H <= 0 || pb->m <= 0 || pb->dh <= 0) return 1;
    if (pb->in_dtype != SAO_F32 && pb->in_dtype != SAO_BF16 && pb->in_dtype != SAO_F64) return 1;
    if (pb->norm != SAO_HISTORY && pb->norm != SAO_PROTOTYPE) return 1;
    return 0;
}

/*
 * Full forward.  S: [B, H, m, dh].  lse (optional): history [B, H, m];
 * prototype [total_rows, H] (rows outside every user or masked get -inf).
 * Returns 0 on success, non-zero on invalid arguments.
 */
int sao_forward(const sao_problem* pb, const void* P, const void* K, const void* V,
                const int32_t* cu, const int32_t* lengths, const uint8_t* mask,
                double* S, double* lse) {
    if (check(pb)) return 1;
    const int B = pb->B, H = pb->H, m = pb->m, dh = pb->dh;
    if (pb->norm == SAO_PROTOTYPE && lse)
        for (int64_t x = 0; x < pb->total_rows * H; ++x) lse[x] = -INFINITY;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            int64_t* rows;
            const int64_t n = valid_rows(pb, cu, lengths, mask, b, &rows);
            double* S_bh = S + ((int64_t)b * H + h) * m * dh;
            if (pb->norm == SAO_HISTORY) {
                double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
                for (int j = 0; j < m; ++j) {
                    double l;
                    history_one(pb, P, K, V, rows, n, b, h, j, s, S_bh + (int64_t)j * dh, &l);
                    if (lse) lse[((int64_t)b * H + h) * m + j] = l;
                }
                free(s);
            } else {
                prototype_bh(pb, P, K, V, rows, n, b, h, S_bh, lse);
            }
            free(rows);
        }
    }
    return 0;
}

/*
 * History axis only: the rows S[b,h,j,:] for n sampled triples bhj[3*t+0..2].
 * out: [n, dh]; lse (optional): [n].  Cost is O(L_b * dh) per sample, so it
 * serves full-size checks where the whole forward would take too long.
 */
int sao_forward_sample(const sao_problem* pb, const void* P, const void* K, const void* V,
                       const int32_t* cu, const int32_t* lengths, const uint8_t* mask,
                       int32_t n, const int32_t* bhj, double* out, double* lse) {
    if (check(pb) || pb->norm != SAO_HISTORY) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < n; ++t) {
        const int b = bhj[3 * t], h = bhj[3 * t + 1], j = bhj[3 * t + 2];
        int64_t* rows;
        const int64_t cnt = valid_rows(pb, cu, lengths, mask, b, &rows);
        double* s = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
        double l;
        history_one(pb, P, K, V, rows, cnt, b, h, j, s, out + (int64_t)t * pb->dh, &l);
        if (lse) lse[t] = l;
        free(s);
        free(rows);
    }
    return 0;
}

/*
 * The materialised assignment matrix of one (b, h): A[j, t] for the user's
 * valid rows t = 0..n-1 in ascending order (the naive path that section 4.4,
 * FlashSA, describes as storing the whole k x n matrix).
 * A: [m, cap]; returns the number of valid rows, or -1 if it exceeds cap.
 */
int64_t sao_assignment(const sao_problem* pb, const void* P, const void* K,
                       const int32_t* cu, const int32_t* lengths, const uint8_t* mask,
                       int32_t b, int32_t h, int64_t cap, double* A) {
    if (check(pb)) return -1;
    int64_t* rows;
    const int64_t n = valid_rows(pb, cu, lengths, mask, b, &rows);
    if (n > cap) {
        free(rows);
        return -1;
    }
    const int m = pb->m;
    for (int j = 0; j < m; ++j)
        for (int64_t t = 0; t < n; ++t) A[(int64_t)j * cap + t] = score(pb, P, K, b, h, j, rows[t]);
    if (pb->norm == SAO_HISTORY) {
        for (int j = 0; j < m; ++j) {
            double M = -INFINITY, Z = 0.0;
            double* a = A + (int64_t)j * cap;
            for (int64_t t = 0; t < n; ++t) if (a[t] > M) M = a[t];
            for (int64_t t = 0; t < n; ++t) Z += exp(a[t] - M);
            for (int64_t t = 0; t < n; ++t) a[t] = exp(a[t] - M) / Z;
        }
    } else {
        for (int64_t t = 0; t < n; ++t) {
            double M = -INFINITY, Z = 0.0;
            for (int j = 0; j < m; ++j) if (A[(int64_t)j * cap + t] > M) M = A[(int64_t)j * cap + t];
            for (int j = 0; j < m; ++j) Z += exp(A[(int64_t)j * cap + t] - M);
            for (int j = 0; j < m; ++j) A[(int64_t)j * cap + t] = exp(A[(int64_t)j * cap + t] - M) / Z;
        }
    }
    free(rows);
    return n;
}

/*
 * Projection in double: out[r, c] = sum_k X[row_r, k] * W[k, c] for the listed
 * rows (rows == NULL: rows 0..nrows-1), columns [c0, c0+nc) of W.
 * X: [*, d_model] (stored dtype), W: [d_model, ldw] (stored dtype).
 * This is the key projection K = X W_K of appendix G.3 (SA FLOPs), unrounded.
 */
int sao_project(const void* X, const void* W, int32_t in_dtype, int32_t d_model, int64_t ldw,
                int64_t nrows, const int64_t* rows, int64_t c0, int64_t nc, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        for (int64_t c = 0; c < nc; ++c) {
            double acc = 0.0;
            for (int k = 0; k < d_model; ++k)
                acc += widen(X, in_dtype, row * d_model + k) * widen(W, in_dtype, (int64_t)k * ldw + c0 + c);
            out[r * nc + c] = acc;
        }
    }
    return 0;
}

/* Number of OpenMP threads the parallel loops above may use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int sao_threads(void) { return omp_get_max_threads(); }
#else
int sao_threads(void) { return 1; }
#endif
