// bw_probe.hip -- HBM bandwidth probes used by the bench to measure the
// ceiling the cross-entropy kernels are held against: a read-only stream
// (every 16-byte vector read once, folded into one value per workgroup so the
// reads cannot be dropped) and a plain copy.  Not part of the cross-entropy
// library; built into its own libce_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct alignas(16) V4 {
    uint32_t w[4];
};

template <int U>
__global__ void __launch_bounds__(256) read_kernel(const V4 *__restrict__ src, int64_t nvec,
                                                   float *__restrict__ out)
{
    float acc = 0.0f;
    const int64_t step = (int64_t)gridDim.x * blockDim.x * U;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < nvec;
         base += step) {
        V4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            r[u] = src[i < nvec ? i : nvec - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc += __uint_as_float(r[u].w[0] ^ r[u].w[1] ^ r[u].w[2] ^ r[u].w[3]) * 0.0f + 1.0f;
    }
    __shared__ float s[256];
    s[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int i = 0; i < (int)blockDim.x; ++i)
            t += s[i];
        out[blockIdx.x] = t;
    }
}

template <int U>
__global__ void __launch_bounds__(256) copy_kernel(V4 *__restrict__ dst, const V4 *__restrict__ src,
                                                   int64_t nvec)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x * U;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < nvec;
         base += step) {
        V4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            if (i < nvec)
                r[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            if (i < nvec)
                dst[i] = r[u];
        }
    }
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from src; out needs `grid` floats.
int probe_read(const void *src, int64_t bytes, int grid, int unroll, float *out, void *stream)
{
    const int64_t nvec = bytes / 16;
    if (!src || !out || nvec < 1 || grid < 1)
        return -1;
    hipStream_t s = (hipStream_t)stream;
    const V4 *p = (const V4 *)src;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(grid), dim3(256), 0, s, p, nvec, out); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(grid), dim3(256), 0, s, p, nvec, out); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(grid), dim3(256), 0, s, p, nvec, out); break;
    case 16: hipLaunchKernelGGL(read_kernel<16>, dim3(grid), dim3(256), 0, s, p, nvec, out); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int probe_copy(void *dst, const void *src, int64_t bytes, int grid, int unroll, void *stream)
{
    const int64_t nvec = bytes / 16;
    if (!src || !dst || nvec < 1 || grid < 1)
        return -1;
    hipStream_t s = (hipStream_t)stream;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(copy_kernel<1>, dim3(grid), dim3(256), 0, s, (V4 *)dst, (const V4 *)src, nvec); break;
    case 4: hipLaunchKernelGGL(copy_kernel<4>, dim3(grid), dim3(256), 0, s, (V4 *)dst, (const V4 *)src, nvec); break;
    case 8: hipLaunchKernelGGL(copy_kernel<8>, dim3(grid), dim3(256), 0, s, (V4 *)dst, (const V4 *)src, nvec); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
