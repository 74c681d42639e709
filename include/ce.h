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
 * Numerics: every row is reduced in fp32 in one pass (running max and a sum
 * of exp2((x - max) * log2 e) rescaled when the max grows); row losses are
 * accumulated in fp64 and the
 * mean/sum is formed in fp64 in a fixed order, so results are bitwise
 * reproducible for a given device and shape.  Gradients are rounded to the
 * storage type with round-to-nearest-even (subnormals kept).  The final sum
 * of a mean/sum runs in the last workgroup of the launch that made the
 * partials, or, during graph capture and for split rows, as a second
 * one-wavefront kernel (the same fixed order, the same bits): the first form
 * takes one integer counter per device and stream in the library's own
 * device memory, zero between calls.
 *
 * Memory and ownership: every pointer is device memory owned by the caller.
 * The library allocates nothing, frees nothing and keeps no pointer after a
 * call returns (its static device memory -- the counters above and the
 * scratch of ce_fwd_noalloc -- is part of the loaded library).  Calls are asynchronous on `stream` (a hipStream_t; NULL is
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

/* Compiled as C++, the enums below have int as their underlying type, so a
 * caller's out-of-range code is a value the checks can reject (without it,
 * C++ leaves an enum holding a value outside its enumerators' range
 * undefined); compiled as C they are plain enums, as always. */
#ifdef __cplusplus
#define CE_INT_ENUM : int
#else
#define CE_INT_ENUM
#endif

/* Storage type of the logits (and of the in-place gradient). */
typedef enum ce_dtype_e CE_INT_ENUM { CE_F32 = 0, CE_F16 = 1, CE_BF16 = 2 } ce_dtype_t;

/* Reduction over rows. */
typedef enum ce_reduction_e CE_INT_ENUM { CE_NONE = 0, CE_MEAN = 1, CE_SUM = 2 } ce_reduction_t;

/* Status codes: 0 is success, negative values are errors. */
enum {
    CE_OK = 0,
    CE_ERR_NULL = -1,        /* a required pointer is NULL */
    CE_ERR_SHAPE = -2,       /* M < 0, V < 1, V > CE_MAX_V, or M*V*size overflows */
    CE_ERR_DTYPE = -3,       /* dtype is not a ce_dtype_t */
    CE_ERR_REDUCTION = -4,   /* reduction is not a ce_reduction_t */
    CE_ERR_WORKSPACE = -5,   /* workspace NULL or too small for a mean / sum, or
                                not 8-byte aligned */
    CE_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
    CE_ERR_ALIGNMENT = -7,   /* a pointer not aligned to its element size, or an
                                output not at the logits' address modulo 16 */
    CE_ERR_ALIAS = -8,       /* an output overlaps another output or an input */
    CE_ERR_SCRATCH = -9      /* ce_fwd_noalloc: the call needs more than the
                                library's static scratch holds */
};

/* Largest supported row length (classes per row). */
#define CE_MAX_V 2147483647LL

/*
 * Bytes of device workspace a call with these arguments can use:
 *  - the mean or sum of ce_fwd / ce_fwd_lse / ce_fwd_bwd_inplace needs
 *    128 KiB (up to 16384 fp64 partial sums, one per workgroup of the
 *    launch, added in a fixed order by the launch's last workgroup or a
 *    one-wavefront kernel);
 *  - few long rows (M <= 128 and rows of at least 256 KiB) are split over
 *    several workgroups when the call gets a workspace of the size returned
 *    here (128 KiB plus up to M * 772 bytes), for every entry point and
 *    every reduction; with less (or NULL, where allowed) each row stays in
 *    one workgroup, with the same results to rounding.
 * Returns 0 when no workspace is used (and for invalid arguments).
 *
 * Its contents need no initialization and are scratch after the call.  A
 * call may be several launches on `stream`, so calls on one stream may share
 * a workspace; calls that may run concurrently need distinct workspaces.
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
 * out and the workspace must not overlap logits or targets (CE_ERR_ALIAS).
 * Returns CE_OK or a CE_ERR_* code.
 */
int ce_fwd(const void *logits, const int64_t *targets, int64_t M, int64_t V,
           ce_dtype_t dtype, ce_reduction_t reduction, float *out,
           void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * forward as ce_fwd (same kernels, plans and bits) without a workspace
 * argument: the scratch its kernels need (the fp64 partial sums of a mean or
 * sum, the statistics of split rows) is a static device array of the library,
 * CE_NOALLOC_SCRATCH_BYTES per GPU, held by every GPU the library runs on until
 * the process ends.  The call allocates nothing (no hipMalloc, no library
 * allocation); its device address is looked up on the first call on each
 * device.
 *
 * The scratch covers every call under the default launch plans.  A call that
 * would need more (only a split forced for tuning through CE_FORCE_SPLIT can)
 * returns CE_ERR_SCRATCH before any HIP call; other argument errors are those
 * of ce_fwd, and none involves a workspace.
 *
 * All calls on one GPU share its scratch and nothing in it needs clearing
 * between calls.  Calls that may run concurrently on one GPU (on different
 * streams, or from different host threads without ordering) race on it and
 * must not overlap; calls on one stream are ordered and safe.
 */
#define CE_NOALLOC_SCRATCH_BYTES 229888 /* 128 KiB + 128 * (64 * 12 + 4) bytes */
int ce_fwd_noalloc(const void *logits, const int64_t *targets, int64_t M,
                   int64_t V, ce_dtype_t dtype, ce_reduction_t reduction,
                   float *out, void *stream);

/*
 * Forward that also saves each row's log-sum-exp, for a later ce_bwd:
 * the loss exactly as ce_fwd (same kernels, same bits) and
 *   lse      [M] fp32, lse_i = max_j x_ij + log sum_j exp(x_ij - max_j x_ij).
 * Keeping this one statistic per row (4 bytes) is what lets a later backward
 * be a single streaming pass that writes the gradient to a buffer of its own:
 * the unfused alternative that "9 Triton kernels in 9 weeks", week 7,
 * contrasts with its in-place fused kernel (there the separate [N, V]
 * gradient tensor is what the fused kernel saves).
 * lse must not overlap any other argument (CE_ERR_ALIAS); NULL is
 * CE_ERR_NULL for M > 0.
 */
int ce_fwd_lse(const void *logits, const int64_t *targets, int64_t M,
               int64_t V, ce_dtype_t dtype, ce_reduction_t reduction,
               float *out, float *lse, void *workspace,
               size_t workspace_bytes, void *stream);

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

/*
 * Backward from a saved log-sum-exp (the split form of the week-7 gradient):
 *   grad_ij = d_i * c * (exp(x_ij - lse_i) - [j == t_i])
 * with c = 1/M for CE_MEAN and 1 otherwise, and d the upstream gradient of
 * the loss: dloss[i] for CE_NONE (one per row loss), dloss[0] for CE_MEAN and
 * CE_SUM (the scalar), or 1 when dloss is NULL.  reduction only selects c and
 * the shape of dloss; no loss is computed and no workspace is used.
 *   logits   [M, V] of dtype, read.
 *   lse      [M] fp32, as written by ce_fwd_lse for the same logits.
 *   grad     [M, V] of dtype, written; it must have the same address modulo
 *            16 bytes as logits (CE_ERR_ALIGNMENT).  grad == logits
 *            overwrites the logits; any other overlap with an argument is
 *            CE_ERR_ALIAS.
 *   workspace, workspace_bytes: optional (NULL, 0); see ce_workspace_bytes.
 * A row whose target is outside [0, V) gets d_i c softmax(x_i), with no
 * one-hot term.  Where p_t > 1/2, 1 - p_t is summed from the other terms of
 * the row (one extra read of that row) so the target's gradient keeps its
 * relative accuracy.
 */
int ce_bwd(const void *logits, const int64_t *targets, const float *lse,
           const float *dloss, int64_t M, int64_t V, ce_dtype_t dtype,
           ce_reduction_t reduction, void *grad, void *workspace,
           size_t workspace_bytes, void *stream);

/*
 * Row softmax or log-softmax in one pass over the row: the fused softmax of
 * "9 Triton kernels in 9 weeks", week 1 (the three memory passes of an
 * unfused softmax folded into one), and the log_softmax that the problem
 * statement of the POPCORNBENCH "Kimi-K2.6 l1_p95" trace applies before the
 * negative log-likelihood:
 *   out_ij = exp(x_ij - lse_i)   (log_softmax == 0)
 *   out_ij = x_ij - lse_i        (log_softmax != 0)
 * in the logits' dtype, rounded to nearest even.  out has the same
 * alignment rule and may be logits (in place), as grad of ce_bwd.
 *   lse      optional [M] fp32 row log-sum-exps (NULL: not written).
 *   workspace, workspace_bytes: optional (NULL, 0); see ce_workspace_bytes.
 * A row that is entirely -inf gives NaN.
 */
int ce_softmax(const void *logits, int64_t M, int64_t V, ce_dtype_t dtype,
               int log_softmax, void *out, float *lse, void *workspace,
               size_t workspace_bytes, void *stream);

/* A static, human-readable name for a status code. */
const char *ce_status_string(int status);

/*
 * The library reads its tuning environment variables once, at its first
 * call: CE_FORCE_PLAN, CE_FORCE_SPLIT, CE_FORCE_NBUF, CE_WAVES_PER_CU,
 * CE_FORCE_GRID, CE_ROW_MAP=interleaved|blocked (kernel mapping and launch
 * overrides), CE_FUSE_MAX_BYTES=N (the in-launch final sum of a mean or sum
 * only for inputs of at most N bytes; 0: never) and CE_LINEAR_GEMM
 * (ce_linear.h).  ce_tuning_reload reads them again; for tuning and tests,
 * and not while other threads call the library.
 */
void ce_tuning_reload(void);

/* Operations ce_plan_describe can describe. */
enum {
    CE_OP_FWD = 0,         /* ce_fwd, ce_fwd_lse */
    CE_OP_FWD_BWD = 1,     /* ce_fwd_bwd_inplace */
    CE_OP_SOFTMAX = 2,     /* ce_softmax, log_softmax == 0 */
    CE_OP_LOG_SOFTMAX = 3, /* ce_softmax, log_softmax != 0 */
    CE_OP_BWD = 4          /* ce_bwd */
};

/*
 * Describes the launch plan a call of operation op (CE_OP_*) with these
 * arguments would use on the current device (kernel mapping, tile, grid)
 * into buf, NUL-terminated, for a 16-byte aligned logits pointer.  Returns
 * CE_OK or an error code (an unknown op is CE_ERR_SHAPE).
 */
int ce_plan_describe(int64_t M, int64_t V, ce_dtype_t dtype,
                     ce_reduction_t reduction, int op, char *buf,
                     size_t buf_len);

#ifdef __cplusplus
}
#endif

#endif /* CE_H_ */
