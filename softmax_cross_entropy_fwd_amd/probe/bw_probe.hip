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

template <int U, int NT>
__global__ void __launch_bounds__(NT) read_kernel(const V4 *__restrict__ src, int64_t nvec,
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
    __shared__ float s[NT];
    s[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int i = 0; i < (int)blockDim.x; ++i)
            t += s[i];
        out[blockIdx.x] = t;
    }
}

// The read with the cross-entropy rows kernel's access pattern: each
// wavefront takes tiles of 64*K contiguous vectors (lane l reads vectors l,
// l + 64, ...), tiles grid-strided over all wavefronts of a persistent grid;
// the next tile's K loads are issued (into a second register set) before the
// current tile is folded, so every wavefront keeps a tile of loads in flight.
// NT: non-temporal loads.
template <int K, bool NT>
__device__ __forceinline__ void load_tile(V4 (&r)[K], const V4 *src, int64_t tile, int64_t nvec,
                                          int lane)
{
#pragma unroll
    for (int k = 0; k < K; ++k) {
        int64_t i = tile * 64 * K + lane + 64 * k;
        i = i < nvec ? i : nvec - 1;
        if constexpr (NT) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[k].w[j] = __builtin_nontemporal_load(&src[i].w[j]);
        } else {
            r[k] = src[i];
        }
    }
}

template <int K, bool NT>
__global__ void __launch_bounds__(256) read_tiles_kernel(const V4 *__restrict__ src, int64_t nvec,
                                                         float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t ntiles = (nvec + 64 * K - 1) / (64 * K);
    int64_t tile = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    uint32_t acc = 0;
    if (tile < ntiles) {
        V4 a[K], b[K];
        load_tile<K, NT>(a, src, tile, nvec, lane);
        for (; tile < ntiles; tile += 2 * nwaves) {
            const int64_t t1 = tile + nwaves < ntiles ? tile + nwaves : tile;
            load_tile<K, NT>(b, src, t1, nvec, lane);
#pragma unroll
            for (int k = 0; k < K; ++k)
                acc ^= a[k].w[0] ^ a[k].w[1] ^ a[k].w[2] ^ a[k].w[3];
            if (tile + nwaves >= ntiles)
                break;
            const int64_t t2 = tile + 2 * nwaves < ntiles ? tile + 2 * nwaves : t1;
            load_tile<K, NT>(a, src, t2, nvec, lane);
#pragma unroll
            for (int k = 0; k < K; ++k)
                acc ^= b[k].w[0] ^ b[k].w[1] ^ b[k].w[2] ^ b[k].w[3];
        }
    }
    // one value per lane so the loads cannot be dropped
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = __uint_as_float(acc & 0x7fffffu);
}

// The read with the streamed forward's pattern: a W-wavefront workgroup
// takes whole rows of row_vecs vectors (rows grid-strided) and reads each in
// chunks of W*64*K vectors with non-temporal loads, every chunk's loads
// issued together and folded before the next chunk's.
template <int W, int K>
__global__ void __launch_bounds__(W * 64) read_rows_kernel(const V4 *__restrict__ src,
                                                          int64_t nrows, int64_t row_vecs,
                                                          float *__restrict__ out)
{
    constexpr int64_t CH = (int64_t)W * 64 * K;
    uint32_t acc = 0;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const V4 *q = src + row * row_vecs;
        for (int64_t c = 0; c < row_vecs; c += CH) {
            V4 r[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                int64_t i = c + threadIdx.x + (int64_t)k * W * 64;
                i = i < row_vecs ? i : row_vecs - 1;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    r[k].w[j] = __builtin_nontemporal_load(&q[i].w[j]);
            }
#pragma unroll
            for (int k = 0; k < K; ++k)
                acc ^= r[k].w[0] ^ r[k].w[1] ^ r[k].w[2] ^ r[k].w[3];
        }
    }
    // one value per lane so the loads cannot be dropped
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = __uint_as_float(acc & 0x7fffffu);
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

// The copy with non-temporal loads and stores (streaming hint).
template <int U>
__global__ void __launch_bounds__(256) copy_nt_kernel(V4 *__restrict__ dst,
                                                      const V4 *__restrict__ src, int64_t nvec)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x * U;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < nvec;
         base += step) {
        V4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            if (i < nvec) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    r[u].w[j] = __builtin_nontemporal_load(&src[i].w[j]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            if (i < nvec) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_nontemporal_store(r[u].w[j], &dst[i].w[j]);
            }
        }
    }
}

// In place, with the access pattern of the fused backward over rows held in
// registers: a W-wavefront workgroup reads a row of W*64*K vectors, waits at
// a barrier, and writes the same vectors back (non-temporal); rows are
// grid-strided.  No arithmetic: the rate is what this pattern alone allows.
template <int W, int K>
__global__ void __launch_bounds__(W * 64) inplace_rows_kernel(V4 *__restrict__ p, int64_t nrows)
{
    constexpr int64_t RV = (int64_t)W * 64 * K;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        V4 *q = p + row * RV;
        V4 r[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            r[k] = q[threadIdx.x + k * W * 64];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_nontemporal_store(r[k].w[j], &q[threadIdx.x + k * W * 64].w[j]);
        }
    }
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from src with `block` (256 or 1024) threads
// per workgroup; out needs `grid` floats.
int probe_read(const void *src, int64_t bytes, int grid, int unroll, int block, float *out,
               void *stream)
{
    const int64_t nvec = bytes / 16;
    if (!src || !out || nvec < 1 || grid < 1 || (block != 256 && block != 1024))
        return -1;
    hipStream_t s = (hipStream_t)stream;
    const V4 *p = (const V4 *)src;
#define PROBE_READ(U, NT) \
    if (unroll == U && block == NT) { \
        hipLaunchKernelGGL((read_kernel<U, NT>), dim3(grid), dim3(NT), 0, s, p, nvec, out); \
        return hipGetLastError() == hipSuccess ? 0 : -6; }
    PROBE_READ(1, 256) PROBE_READ(4, 256) PROBE_READ(8, 256) PROBE_READ(16, 256)
    PROBE_READ(1, 1024) PROBE_READ(2, 1024) PROBE_READ(4, 1024) PROBE_READ(8, 1024)
#undef PROBE_READ
    return -1;
}

// The rows-kernel pattern read (read_tiles_kernel): tiles of 64*k vectors,
// k = 8 or 16; nt != 0 for non-temporal loads; 256 threads per workgroup, out
// needs 256 * grid floats.
int probe_read_tiles(const void *src, int64_t bytes, int grid, int k, int nt, float *out,
                     void *stream)
{
    const int64_t nvec = bytes / 16;
    if (!src || !out || nvec < 1 || grid < 1)
        return -1;
    hipStream_t s = (hipStream_t)stream;
    const V4 *p = (const V4 *)src;
#define PROBE_TILES(K, N) \
    if (k == K && (nt != 0) == N) { \
        hipLaunchKernelGGL((read_tiles_kernel<K, N>), dim3(grid), dim3(256), 0, s, p, nvec, out); \
        return hipGetLastError() == hipSuccess ? 0 : -6; }
    PROBE_TILES(8, false) PROBE_TILES(16, false) PROBE_TILES(8, true) PROBE_TILES(16, true)
#undef PROBE_TILES
    return -1;
}

// The streamed-forward pattern read (read_rows_kernel): rows of row_bytes (a
// multiple of 16 dividing bytes), workgroups of W = 4, 8 or 16 wavefronts,
// chunks of W*64*K vectors (K = 4 or 8); out needs W * 64 * grid floats.
int probe_read_rows(const void *src, int64_t bytes, int64_t row_bytes, int W, int K, int grid,
                    float *out, void *stream)
{
    if (!src || !out || grid < 1 || row_bytes < 16 || row_bytes % 16 || bytes % row_bytes)
        return -1;
    const int64_t nrows = bytes / row_bytes, row_vecs = row_bytes / 16;
    hipStream_t s = (hipStream_t)stream;
    const V4 *p = (const V4 *)src;
#define PROBE_ROWS(WW, KK) \
    if (W == WW && K == KK) { \
        hipLaunchKernelGGL((read_rows_kernel<WW, KK>), dim3(grid), dim3(WW * 64), 0, s, p, nrows, \
                           row_vecs, out); \
        return hipGetLastError() == hipSuccess ? 0 : -6; }
    PROBE_ROWS(16, 4) PROBE_ROWS(8, 4) PROBE_ROWS(4, 4) PROBE_ROWS(16, 8) PROBE_ROWS(8, 8)
#undef PROBE_ROWS
    return -1;
}

// unroll 1, 4, 8: plain copy; 101, 102, 104: non-temporal copy unrolled 1, 2, 4.
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
    case 104: hipLaunchKernelGGL(copy_nt_kernel<4>, dim3(grid), dim3(256), 0, s, (V4 *)dst, (const V4 *)src, nvec); break;
    case 102: hipLaunchKernelGGL(copy_nt_kernel<2>, dim3(grid), dim3(256), 0, s, (V4 *)dst, (const V4 *)src, nvec); break;
    case 101: hipLaunchKernelGGL(copy_nt_kernel<1>, dim3(grid), dim3(256), 0, s, (V4 *)dst, (const V4 *)src, nvec); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Rewrite `bytes` in place, rows of W*64*K vectors (W = 16, K = 16 or 8) held
// in registers between the read and the write; bytes must be a multiple of
// the row size.
int probe_inplace_rows(void *p, int64_t bytes, int W, int K, int grid, void *stream)
{
    const int64_t rv = (int64_t)W * 64 * K;
    if (!p || grid < 1 || bytes < 16 * rv || (bytes / 16) % rv || bytes % 16)
        return -1;
    const int64_t nrows = bytes / 16 / rv;
    hipStream_t s = (hipStream_t)stream;
    if (W == 16 && K == 16)
        hipLaunchKernelGGL((inplace_rows_kernel<16, 16>), dim3(grid), dim3(1024), 0, s, (V4 *)p, nrows);
    else if (W == 16 && K == 8)
        hipLaunchKernelGGL((inplace_rows_kernel<16, 8>), dim3(grid), dim3(1024), 0, s, (V4 *)p, nrows);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
