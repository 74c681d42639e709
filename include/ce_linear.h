/*
 * ce_linear.h -- linear + cross-entropy on MI355X (gfx950): the C ABI.
 *
 * The operation: the logits of an lm_head projection,
 *     z = H W^T,   H [M, D] hidden states, W [V, D] weight (bf16),
 * fed to the row-wise softmax cross-entropy of ce.h (loss_i = lse(z_i) -
 * z[i, t_i], reduced by none, mean or sum), without ever holding the whole
 * [M, V] logits.  This is the fused linear + cross-entropy of "9 Triton
 * kernels in 9 weeks", week 8 (the lm_head projection chunked into the loss
 * to cut activation memory).
 *
 * Two ways to the logits, the same numerics (bf16 products, fp32
 * accumulation, fp32 row arithmetic):
 *   - the library's own matrix-core kernels (bf16 MFMA), when D % 8 == 0,
 *     D <= 2^20 and H and W sit on 16-byte boundaries: the forward forms
 *     256 x 256 tiles of z and folds each into per-row statistics (max and
 *     sum of exp over each 128 vocabulary rows, the target left out) in the
 *     same kernel, so no logits are written at all;
 *   - otherwise (or with the environment variable CE_LINEAR_GEMM=library)
 *     rocBLAS GEMMs over vocabulary chunks of C columns, each chunk's fp32
 *     logits folded into per-row statistics before the next overwrites them.
 * The backward takes the vocabulary in chunks of C columns, recomputes each
 * chunk's logits, writes their gradient
 *     G = (softmax(z) - onehot(t)) * c     (c = 1/M for mean, 1 otherwise)
 * in bf16 ([M][C], from a matrix-core kernel or a row kernel), and accumulates
 * dH = G W and dW = G^T H (fp32 outputs) with two rocBLAS GEMMs per chunk.
 * The per-row combine has the numerics of ce.h (the target left out of the
 * sums so dominant targets keep their relative accuracy, fp64 fixed-order
 * mean / sum).
 *
 * Memory: every pointer is device memory owned by the caller.  Where
 * rocBLAS runs (the backward, the library forward) the library creates one
 * rocBLAS handle per device and stream on first use (rocBLAS allocates its
 * own small workspace then) and keeps it until the process ends; a handle
 * serves one call at a time, so calls on different streams do not wait for
 * each other on the host.  Everything else lives in the caller's workspace.
 * Calls are asynchronous on `stream` (a hipStream_t); argument errors return
 * before any launch.  Calls that may run concurrently need distinct
 * workspaces.
 *
 * Layout: H row-major [M, D], W row-major [V, D] (the nn.Linear weight
 * layout), both bf16 and 2-byte aligned; targets int64 [M]; dH row-major
 * [M, D] fp32; dW row-major [V, D] fp32.  M, D and V must fit in int32.
 * Status codes are those of ce.h.
 */
#ifndef CE_LINEAR_H_
#define CE_LINEAR_H_

#include <stddef.h>
#include <stdint.h>

#include "ce.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The vocabulary chunk (columns per chunk) the calls use for these sizes
 * when given chunk == 0: a multiple of 256, at least 1024, with the fp32
 * logits chunk (M * C * 4 bytes) near 128 MiB.  A given chunk is rounded up
 * to a multiple of 256; no chunk exceeds V rounded up to 256.
 */
int64_t ce_linear_chunk(int64_t M, int64_t D, int64_t V, int64_t chunk);

/*
 * Workspace bytes ce_linear_fwd / ce_linear_fwd_bwd need for these sizes and
 * chunk (0 = the default): the larger of the library path's fp32 logits and
 * bf16 gradient chunks (M * C * 6 bytes) with its chunk statistics, and the
 * matrix-core path's statistics (8 bytes per token and 128 vocabulary rows)
 * with its bf16 gradient chunk (M * C * 2 bytes); then per-row buffers.  0 for invalid
 * sizes.  Contents need no initialization.
 */
size_t ce_linear_workspace_bytes(int64_t M, int64_t D, int64_t V, int64_t chunk);

/*
 * Forward: out receives the M row losses (none) or one value (mean, sum);
 * lse (optional, [M] fp32) the rows' log-sum-exps.
 */
int ce_linear_fwd(const void *hidden, const void *weight, const int64_t *targets,
                  int64_t M, int64_t D, int64_t V, ce_reduction_t reduction,
                  float *out, float *lse, int64_t chunk, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * Forward and backward: the loss as ce_linear_fwd, and the gradients of that
 * loss, dhidden [M, D] and dweight [V, D] (fp32, overwritten).  No output may
 * overlap an input, another output or the workspace (CE_ERR_ALIAS).
 */
int ce_linear_fwd_bwd(const void *hidden, const void *weight, const int64_t *targets,
                      int64_t M, int64_t D, int64_t V, ce_reduction_t reduction,
                      float *out, float *lse, float *dhidden, float *dweight,
                      int64_t chunk, void *workspace, size_t workspace_bytes,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CE_LINEAR_H_ */
