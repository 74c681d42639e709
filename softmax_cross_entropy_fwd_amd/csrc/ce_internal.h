// ce_internal.h -- host-side view of the compiled kernel instances.
#pragma once

namespace cek {

enum Kind : int { KIND_ROWS = 0, KIND_WG = 1, KIND_STREAM = 2, KIND_WSTREAM = 3 };

struct KernelRef {
    const void *fn;   // host stub of a __global__ instance, or nullptr
    int block;        // threads per workgroup it was compiled for
};

// (kind, a, b): rows (G lanes per row, K vectors per lane), wg (W waves,
// K vectors per lane), stream (W waves, K vectors per lane per chunk) or
// wstream (a = 1 wave per row, K vectors per lane per chunk; forward only).
// exact: every row window is exactly the tile (aligned rows of G*K or
// W*64*K vectors); no stream kernel is exact.  nbuf: row buffers per lane of
// the rows kernel (1 or 2).
KernelRef get_kernel_f32(int kind, int a, int b, bool bwd, bool exact, int nbuf);
KernelRef get_kernel_f16(int kind, int a, int b, bool bwd, bool exact, int nbuf);
KernelRef get_kernel_bf16(int kind, int a, int b, bool bwd, bool exact, int nbuf);

const void *empty_reduce_fn();

}  // namespace cek
