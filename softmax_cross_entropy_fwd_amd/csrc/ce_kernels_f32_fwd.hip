// f32 kernel instances: forward.
#define CE_DT DT_F32
#define CE_PART 0
#define CE_GET_KERNEL get_kernel_f32_fwd
#include "ce_kernels_inst.h"

namespace cek {

// M == 0: the mean of no rows is NaN, their sum is 0.
__global__ void empty_reduce_kernel(float *out, float value)
{
    if (threadIdx.x == 0)
        out[0] = value;
}

const void *empty_reduce_fn() { return (const void *)&empty_reduce_kernel; }

// Second-kernel form of the final sum of a mean / sum (one wavefront).
__global__ void __launch_bounds__(64) sum_partials_kernel(Params p, unsigned nunits)
{
    const double total = sum_partials(p.partials, nunits, threadIdx.x);
    if (threadIdx.x == 0)
        p.out[0] = (float)(total * p.out_scale);
}

const void *sum_partials_fn() { return (const void *)&sum_partials_kernel; }

}  // namespace cek
