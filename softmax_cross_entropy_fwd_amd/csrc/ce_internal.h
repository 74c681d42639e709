// ce_internal.h -- host-side view of the compiled kernel instances.
#pragma once

namespace cek {

enum Kind : int { KIND_ROWS = 0, KIND_WG = 1, KIND_STREAM = 2 };

struct KernelRef {
    const void *fn;   // host stub of a __global__ instance, or nullptr
    int block;        // threads per workgroup it was compiled for
};

// (kind, a, b): rows (G lanes per row, K vectors per lane), wg (W waves,
// K vectors per lane) or stream (W waves, K vectors per lane per chunk).
KernelRef get_kernel_f32(int kind, int a, int b, bool bwd);
KernelRef get_kernel_f16(int kind, int a, int b, bool bwd);
KernelRef get_kernel_bf16(int kind, int a, int b, bool bwd);

const void *empty_reduce_fn();

}  // namespace cek
