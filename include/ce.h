/*
 * ce.h -- row-wise softmax cross-entropy on MI355X (gfx950): the C ABI.
 *
 * The operation (all entry points):
 *   For a row-major logits matrix x[M, V] and integer targets t[M],
 *     lse_i  = log sum_j exp(x_ij)                  (log-sum-exp of row i)
 *     loss_i = lse_i - x[i, t_i]
 *   reduced by none (the M row losses), mean (sum / M) or sum.
 *   This is the cross-entropy of the POPCORNBENCH "Kimi-K2.6 l1_p95" trace
 *   (problem statement: log_softmax, negative log-likelihood of the target,
 *   mean over the batch) and of loss_kernel in the Triton issue "Cross
 *   Entropy Loss performance issue" (per-row output log(sumexp) + max - x_t).
 *
 *   The fused backward ("9 Triton kernels in 9 weeks", week 7: forward and
 *   backward in one kernel, gradient written over the logits buffer) writes
 *     g_ij = (softmax(x_i)_j - [j == t_i]) * c
 *   in place over x, with c = 1/M for mean and c = 1 for sum and none (the
 *   gradient of the returned loss, or of the sum of the row losses).
 *
 * Numerics: every row is reduced in fp32 (online max, then sum of
 * exp2((x - max) * log2 e)); row losses are accumulated in fp64 and the
 * mean/sum is formed in fp64 in a fixed order, so results are bitwise
 * reproducible for a given device and shape.  Gradients are rounded to the
 * storage type with round-to-nearest-even (subnormals kept).
 *
 * Memory and ownership: every pointer is device memory owned by the caller.
 * The library allocates nothing, frees nothing and keeps no pointer after a
 * call returns.  Calls are asynchronous on `stream` (a hipStream_t; NULL is
 * the null stream); argument errors are returned synchronously before any
 * launch.
 *
 * Layout: logits are row-major and contiguous (row stride V elements); any
 * element-aligned base pointer is accepted.  Targets are int64 [M].
 *
 * Target values outside [0, V) do not fault and are not checked on the host:
 * that row's loss is NaN (so the mean and sum are NaN) and its gradient row is
 * softmax * c with no one-hot term.
 */
#ifndef CE_H_
#define CE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of the logits (and of the in-place gradient). */
typedef enum { CE_F32 = 0, CE_F16 = 1, CE_BF16 = 2 } ce_dtype_t;

/* Reduction over rows. */
typedef enum { CE_NONE = 0, CE_MEAN = 1, CE_SUM = 2 } ce_reduction_t;

/* Status codes: 0 is success, negative values are errors. */
enum {
    CE_OK = 0,
    CE_ERR_NULL = -1,        /* a required pointer is NULL */
    CE_ERR_SHAPE = -2,       /* M < 0, V < 1, V > CE_MAX_V, or M*V*size overflows */
    CE_ERR_DTYPE = -3,       /* dtype is not a ce_dtype_t */
    CE_ERR_REDUCTION = -4,   /* reduction is not a ce_reduction_t */
    CE_ERR_WORKSPACE = -5,   /* workspace NULL, too small or not 8-byte aligned */
    CE_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
    CE_ERR_ALIGNMENT = -7,   /* logits not aligned to its element size */
    CE_ERR_ALIAS = -8        /* in-place logits overlap targets, output or workspace */
};

/* Largest supported row length (classes per row). */
#define CE_MAX_V 2147483647LL

/*
 * Bytes of device workspace ce_fwd / ce_fwd_bwd_inplace need for these
 * arguments: 0 for CE_NONE and for M == 0, otherwise a fixed 33 KiB
 * (a ticket word and up to 4096 fp64 partial sums).
 *
 * The workspace must be zero-filled before its first use; every call leaves
 * it zero-filled again, so one workspace can be reused by successive calls on
 * one stream.  Calls that may run concurrently need distinct workspaces.
 * Returns 0 for invalid arguments as well.
 */
size_t ce_workspace_bytes(int64_t M, int64_t V, ce_dtype_t dtype,
                          ce_reduction_t reduction);

/*
 * Forward: the loss of every row, reduced.
 *   logits   [M, V] of dtype, read only.
 *   targets  [M] int64.
 *   out      CE_NONE: [M] fp32 row losses; CE_MEAN / CE_SUM: one fp32.
 *            M == 0 writes NaN (mean) or 0 (sum) and nothing for none.
 *   workspace, workspace_bytes: see ce_workspace_bytes (NULL, 0 for none).
 *   stream   hipStream_t the work is queued on.
 * Returns CE_OK or a CE_ERR_* code.
 */
int ce_fwd(const void *logits, const int64_t *targets, int64_t M, int64_t V,
           ce_dtype_t dtype, ce_reduction_t reduction, float *out,
           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Fused forward + backward in place: computes the loss exactly as ce_fwd
 * (into loss_out) and overwrites logits with the gradient of that loss,
 * (softmax - onehot) * c, in the same dtype.  logits must not overlap
 * targets, loss_out or the workspace (CE_ERR_ALIAS).
 */
int ce_fwd_bwd_inplace(void *logits, const int64_t *targets, int64_t M,
                       int64_t V, ce_dtype_t dtype, ce_reduction_t reduction,
                       float *loss_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* A static, human-readable name for a status code. */
const char *ce_status_string(int status);

/*
 * Describes the launch plan a call with these arguments would use on the
 * current device (kernel mapping, tile, grid) into buf, NUL-terminated.
 * fwd_bwd selects the in-place variant.  Returns CE_OK or an error code.
 */
int ce_plan_describe(int64_t M, int64_t V, ce_dtype_t dtype,
                     ce_reduction_t reduction, int fwd_bwd, char *buf,
                     size_t buf_len);

#ifdef __cplusplus
}
#endif

#endif /* CE_H_ */
