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

const void *stats_kernel_fn();    // one wavefront per row, 256 threads
const void *finish_kernel_fn();   // one wavefront per row, 256 threads
const void *grad_kernel_fn();     // one wavefront per row, 256 threads
const void *zero_kernel_fn();     // (float *p, int64_t n), 256 threads

}  // namespace lce
