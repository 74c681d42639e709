// lce_internal.h -- kernels of the linear + cross-entropy path (host view).
#pragma once

#include <cstdint>

namespace lce {

// One vocabulary chunk of the logits, [M, ldc] fp32, and what the kernels
// read and write around it.
struct LceParams {
    const float *L;           // [M, ldc] logits chunk (columns v0 .. v0 + vn)
    uint16_t *G;              // [M, ldc] bf16 gradient chunk
    const int64_t *targets;   // [M]
    int64_t M;
    int64_t V;
    int64_t v0;               // first vocabulary column of the chunk
    int ldc;                  // row stride of L and G (elements), a multiple of 8
    int vn;                   // columns of this chunk
    int chunk_index;
    int nchunks;
    float *stats;             // [M, nchunks, 2] chunk (max, sum), the target left out
    float *rowx;              // [M] target logits
    float *lse;               // [M] row log-sum-exps (workspace)
    float *gt;                // [M] the target's gradient
    float *lse_out;           // optional [M]
    float *out;               // [M] losses (none) or null
    double *partials;         // [M] losses to add (mean / sum) or null
    float c;                  // gradient scale
};

// The matrix-core path (lce_mfma.hip): tiles of z^T = W H^T, 256 vocabulary
// rows x 256 tokens per 256-thread workgroup; a persistent grid (any size,
// a multiple of 8 keeps each workgroup's tiles on its XCD's L2) walks the
// ntiles_v * ntiles_t tiles.
// Needs D % 8 == 0 and H, W on 16-byte boundaries.
struct MfmaParams {
    const uint16_t *H;        // [M, D] bf16
    const uint16_t *W;        // [V, D] bf16 (the launch covers rows v0 .. v0 + vn)
    const int64_t *targets;   // [M]
    int64_t M, D, V;
    int64_t v0;
    int vn;
    int ntiles_v, ntiles_t;
    // forward: per token, (max, sum) of each 128 vocabulary rows with the
    // target left out, [M][nhalf][2], entries half0 + 2 tv + (0, 1); the
    // target's logit in rowx
    float *stats;
    int nhalf;
    int half0;
    float *rowx;
    // backward: the row statistics and the gradient chunk
    const float *lse;         // [M]
    const float *gt;          // [M] the target's gradient
    float c;                  // gradient scale, > 0
    uint16_t *G;              // [M][ldg] bf16, columns 0 .. vn
    int64_t ldg;              // row stride of G (elements), a multiple of 8, >= vn
};

const void *mfma_stats_kernel_fn();   // MfmaParams, 256 threads
const void *mfma_grad_kernel_fn();    // MfmaParams, 256 threads

const void *stats_kernel_fn();    // one wavefront per row, 256 threads
const void *finish_kernel_fn();   // one wavefront per row, 256 threads
const void *grad_kernel_fn();     // one wavefront per row, 256 threads
const void *zero_kernel_fn();     // (float *p, int64_t n), 256 threads

}  // namespace lce
