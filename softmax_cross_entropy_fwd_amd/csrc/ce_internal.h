// ce_internal.h -- host-side view of the compiled kernel instances.
#pragma once

namespace cek {

// KIND_WG2: one row per 8-wave workgroup held to 128 VGPRs, two workgroups per CU.
enum Kind : int { KIND_ROWS = 0, KIND_WG = 1, KIND_STREAM = 2, KIND_WSTREAM = 3, KIND_WG2 = 4 };

struct KernelRef {
    const void *fn;   // host stub of a __global__ instance, or nullptr
    int block;        // threads per workgroup it was compiled for
};

// op: EPI_NONE (forward), EPI_GRAD (fused in-place backward), EPI_SOFTMAX,
// EPI_LOGSOFTMAX or EPI_LSE_GRAD (backward from a given log-sum-exp).
// (kind, a, b): rows (G lanes per row, K vectors per lane), wg (W waves, K
// vectors per lane), stream (W waves, K vectors per lane per chunk) or
// wstream (a = 1 wave per row, K vectors per lane per chunk; forward only).
// exact: every row window is exactly the tile (aligned rows of G*K or
// W*64*K vectors).  nbuf: row buffers per lane of the rows kernel (1 or 2;
// 17 or 18 for 16-wave workgroups).  Each unit answers its own operations:
// _fwd EPI_NONE, _grad EPI_GRAD, _aux the rest; others get a null KernelRef.
KernelRef get_kernel_f32_fwd(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_f32_grad(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_f32_aux(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_f16_fwd(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_f16_grad(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_f16_aux(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_bf16_fwd(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_bf16_grad(int op, int kind, int a, int b, bool exact, int nbuf);
KernelRef get_kernel_bf16_aux(int op, int kind, int a, int b, bool exact, int nbuf);

// Split rows (several workgroups per row): slice statistics, the forward's
// per-row finish (64 threads), the epilogue per operation (indexed by EPI_*,
// null for EPI_NONE), the target fix of the backward from a given lse.
// Slices are streamed in chunks of kSplitChunk window vectors by 256 threads.
constexpr int kSplitChunk = 1024;
struct SplitKernels {
    const void *stats;
    const void *finish;
    const void *epi[5];
    const void *fix;
};
SplitKernels split_kernels_f32();
SplitKernels split_kernels_f16();
SplitKernels split_kernels_bf16();

const void *empty_reduce_fn();
const void *sum_partials_fn();

// CE_LINEAR_GEMM=library, as read with the other tuning variables.
bool tuning_linear_library();

}  // namespace cek
