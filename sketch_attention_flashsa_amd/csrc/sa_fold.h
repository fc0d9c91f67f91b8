// sa_fold.h -- keys folded into the prototypes (sa_fused_proj.hip).
#pragma once

#include "sa_internal.h"

namespace sa {

// out[h][j][e] = bf16(c * sum_k P[h][j][k] * W[e][h dh + k]) for h < H, j < m,
// e < d_model: the prototypes of head h moved through W_K,h^T, so that
// P_h (X W_K,h)^T = out_h X^T (appendix G.2.1's reordering, for SA).
// P [H, m, dh], W [d_model, H dh] and out [H, m, d_model] are bf16; the sum is
// fp32 (MFMA) and is rounded once.  Needs m and d_model multiples of 16 and
// dh a multiple of 32 (else hipErrorInvalidValue); the folded path's shapes
// (one head, dh = d_model = 128, m a multiple of 256) always are.
hipError_t launch_fold_keys(const bf16* P, const bf16* W, int H, int m, int dh, int d_model, float c, bf16* out,
                            hipStream_t s);

}  // namespace sa
