// lce_api.hip -- the C ABI of linear + cross-entropy: argument checks, the
// choice of the matrix-core path (lce_mfma.hip) or the library GEMMs
// (rocBLAS) with the row kernels (lce_kernels.hip), the chunk loop and the
// launches.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <utility>

#include "ce.h"
#include "ce_device.h"
#include "ce_internal.h"
#include "ce_linear.h"
#include "lce_internal.h"

namespace {

constexpr int64_t kChunkAlign = 256;         // columns
// Default chunk: its fp32 logits take about 128 MiB, half the last-level
// cache, so the statistics and gradient passes mostly read what the GEMM just
// wrote (measured on the 4096 x 4096 x 131072 workload: 8192 columns, forward
// 3.79 ms and forward + backward 15.5 ms, against 4.26 / 16.4 ms with 43520).
constexpr int64_t kChunkBytes = 128LL << 20;
constexpr int64_t kMinChunk = 1024;

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

int64_t chunk_for(int64_t M, int64_t V, int64_t chunk)
{
    const int64_t vmax = (V + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    int64_t C;
    if (chunk > 0) {
        C = (chunk + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    } else {
        const int64_t per_col = 4 * (M > 0 ? M : 1);   // fp32 logits
        C = kChunkBytes / per_col / kChunkAlign * kChunkAlign;
        if (C < kMinChunk)
            C = kMinChunk;
    }
    return C < vmax ? C : vmax;
}

constexpr int64_t kMfmaTile = 256;   // vocabulary rows and tokens per matrix-core tile

// Statistics entries per row of the matrix-core forward: one per 128
// vocabulary rows.
int64_t mfma_halves(int64_t V) { return 2 * ((V + kMfmaTile - 1) / kMfmaTile); }

// Workspace layout (offsets in bytes, each 256-aligned).  The head holds
// either path's buffers -- library GEMMs: the fp32 logits chunk L, the bf16
// gradient chunk G [M][C] and the chunk statistics; matrix-core kernels: the
// per-128-rows statistics and the gradient chunk Gm [M][C] -- and the
// per-row buffers follow the larger of the two.
struct Layout {
    size_t L, G, stats, stats_m, Gm, rowx, lse, gt, partials, total;
};

Layout layout(int64_t M, int64_t V, int64_t C, int64_t nch)
{
    Layout l;
    size_t o = 0;
    l.L = o;
    o += align256((size_t)M * C * 4);
    l.G = o;
    o += align256((size_t)M * C * 2);
    l.stats = o;
    o += align256((size_t)M * nch * 8);
    size_t om = 0;
    l.stats_m = om;
    om += align256((size_t)M * mfma_halves(V) * 8);
    l.Gm = om;
    om += align256((size_t)M * C * 2);
    if (om > o)
        o = om;
    l.rowx = o;
    o += align256((size_t)M * 4);
    l.lse = o;
    o += align256((size_t)M * 4);
    l.gt = o;
    o += align256((size_t)M * 4);
    l.partials = o;
    o += align256((size_t)M * 8);
    l.total = o;
    return l;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || !na || !nb)
        return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// rocBLAS handles, one per (device, stream): a handle stays bound to its
// stream and serves one call at a time (its own mutex, held while that call
// enqueues its GEMMs), so calls on different streams never wait for each
// other on the host.  Created on first use, kept until the process ends.
struct Blas {
    rocblas_handle h = nullptr;
    std::mutex mu;
};
std::mutex g_map_mu;   // guards g_blas and g_cus
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Blas>> g_blas;
std::map<int, int> g_cus;

Blas *blas_for(int dev, hipStream_t st)
{
    std::lock_guard<std::mutex> lk(g_map_mu);
    std::unique_ptr<Blas> &slot = g_blas[{dev, st}];
    if (!slot) {
        std::unique_ptr<Blas> b(new Blas);
        if (rocblas_create_handle(&b->h) != rocblas_status_success)
            return nullptr;
        if (rocblas_set_stream(b->h, st) != rocblas_status_success) {
            rocblas_destroy_handle(b->h);
            return nullptr;
        }
        slot = std::move(b);
    }
    return slot.get();
}

// The device's compute units (the persistent forward's grid), 0 on error.
int cu_count(int dev)
{
    std::lock_guard<std::mutex> lk(g_map_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end())
        return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    g_cus[dev] = n;
    return n;
}

// C[m x n] (row-major, ldc) = op(A) op(B) + beta C with bf16 A, B and fp32
// C, through rocBLAS's column-major interface (C^T = op(B)^T op(A)^T).
bool gemm_rm(rocblas_handle h, bool ta, bool tb, int m, int n, int k, const void *A, int lda,
             const void *B, int ldb, float beta, float *C, int ldc)
{
    const float alpha = 1.0f;
    return rocblas_gemm_ex(h, tb ? rocblas_operation_transpose : rocblas_operation_none,
                           ta ? rocblas_operation_transpose : rocblas_operation_none, n, m, k,
                           &alpha, B, rocblas_datatype_bf16_r, ldb, A, rocblas_datatype_bf16_r, lda,
                           &beta, C, rocblas_datatype_f32_r, ldc, C, rocblas_datatype_f32_r, ldc,
                           rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                           rocblas_gemm_flags_none) == rocblas_status_success;
}

bool launch(const void *fn, unsigned grid, unsigned block, void **args, hipStream_t st)
{
    return hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, st) == hipSuccess;
}

int run(const void *H, const void *W, const int64_t *targets, int64_t M, int64_t D, int64_t V,
        int reduction, float *out, float *lse, float *dH, float *dW, int64_t chunk, void *ws,
        size_t ws_bytes, void *stream, bool bwd)
{
    if (reduction != CE_NONE && reduction != CE_MEAN && reduction != CE_SUM)
        return CE_ERR_REDUCTION;
    if (M < 0 || D < 1 || V < 1 || M > INT_MAX || D > INT_MAX || V > INT_MAX || chunk < 0)
        return CE_ERR_SHAPE;
    const int64_t C = chunk_for(M, V, chunk);
    const int64_t nch = (V + C - 1) / C;
    const Layout lay = layout(M, V, C, nch);
    hipStream_t st = (hipStream_t)stream;
    const bool reduced = reduction != CE_NONE;
    if (M == 0) {
        if (reduced && !out)
            return CE_ERR_NULL;
        if (bwd && !dW)
            return CE_ERR_NULL;
    } else {
        if (!H || !W || !targets || !out || (bwd && (!dH || !dW)))
            return CE_ERR_NULL;
        if ((uintptr_t)H % 2 || (uintptr_t)W % 2 || (uintptr_t)targets % 8 || (uintptr_t)out % 4 ||
            (uintptr_t)lse % 4 || (uintptr_t)dH % 4 || (uintptr_t)dW % 4)
            return CE_ERR_ALIGNMENT;
        if (!ws || ws_bytes < lay.total || (uintptr_t)ws % 16)
            return CE_ERR_WORKSPACE;
        const size_t hb = (size_t)M * D * 2, wb = (size_t)V * D * 2;
        const struct {
            const void *p;
            size_t n;
        } outs[] = {{out, reduced ? 4 : (size_t)M * 4}, {lse, (size_t)M * 4},
                    {dH, bwd ? (size_t)M * D * 4 : 0}, {dW, bwd ? (size_t)V * D * 4 : 0},
                    {ws, lay.total}},
          ins[] = {{H, hb}, {W, wb}, {targets, (size_t)M * 8}};
        for (int i = 0; i < 5; ++i) {
            for (int j = i + 1; j < 5; ++j)
                if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                    return CE_ERR_ALIAS;
            for (int j = 0; j < 3; ++j)
                if (overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n))
                    return CE_ERR_ALIAS;
        }
    }

    if (M == 0) {
        if (bwd) {
            int64_t n = V * D;
            void *za[] = {&dW, &n};
            if (!launch(lce::zero_kernel_fn(), 1024, 256, za, st))
                return CE_ERR_HIP;
        }
        if (reduced) {
            float value = reduction == CE_MEAN ? __builtin_nanf("") : 0.0f;
            void *args[] = {&out, &value};
            if (!launch(cek::empty_reduce_fn(), 1, 64, args, st))
                return CE_ERR_HIP;
        }
        return CE_OK;
    }

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return CE_ERR_HIP;

    // The logits on this library's matrix-core kernels when the rows are
    // 16-byte vectors (D % 8 == 0, H and W on 16-byte boundaries) and a
    // 256-row tile's bytes fit the kernels' 32-bit buffer offsets (D <=
    // 2^20); else, or with CE_LINEAR_GEMM=library (comparisons), rocBLAS.
    const int64_t tiles = ((V + kMfmaTile - 1) / kMfmaTile) * ((M + kMfmaTile - 1) / kMfmaTile);
    const bool mfma = D % 8 == 0 && D <= (int64_t(1) << 20) && (uintptr_t)H % 16 == 0 &&
                      (uintptr_t)W % 16 == 0 && tiles <= INT_MAX &&
                      !cek::tuning_linear_library();
    // rocBLAS serves the library forward and the backward's dH and dW
    rocblas_handle h = nullptr;
    std::unique_lock<std::mutex> blas_lock;
    if (!mfma || bwd) {
        Blas *b = blas_for(dev, st);
        if (!b)
            return CE_ERR_HIP;
        blas_lock = std::unique_lock<std::mutex>(b->mu);
        h = b->h;
    }

    char *base = (char *)ws;
    lce::LceParams q;
    q.L = (const float *)(base + lay.L);
    q.G = (uint16_t *)(base + lay.G);
    q.targets = targets;
    q.M = M;
    q.V = V;
    q.ldc = (int)C;
    q.nchunks = (int)nch;
    q.stats = (float *)(base + lay.stats);
    q.rowx = (float *)(base + lay.rowx);
    q.lse = (float *)(base + lay.lse);
    q.gt = (float *)(base + lay.gt);
    q.lse_out = lse;
    q.out = reduced ? nullptr : out;
    q.partials = reduced ? (double *)(base + lay.partials) : nullptr;
    q.c = reduction == CE_MEAN ? (float)(1.0 / (double)M) : 1.0f;
    const unsigned row_grid = (unsigned)((M + 3) / 4);
    const int m = (int)M, d = (int)D;
    float *Lw = (float *)(base + lay.L);
    lce::MfmaParams mp{};
    mp.H = (const uint16_t *)H;
    mp.W = (const uint16_t *)W;
    mp.targets = targets;
    mp.M = M;
    mp.D = D;
    mp.V = V;
    mp.ntiles_t = (int)((M + kMfmaTile - 1) / kMfmaTile);
    mp.rowx = q.rowx;
    mp.lse = q.lse;
    mp.gt = q.gt;
    mp.c = q.c;
    mp.G = (uint16_t *)(base + lay.Gm);
    mp.ldg = C;
    if (mfma) {
        // forward: every tile's statistics in one launch over all of V, a
        // persistent workgroup per compute unit
        const int cus = cu_count(dev);
        if (cus < 1)
            return CE_ERR_HIP;
        mp.v0 = 0;
        mp.vn = (int)V;
        mp.ntiles_v = (int)((V + kMfmaTile - 1) / kMfmaTile);
        mp.stats = (float *)(base + lay.stats_m);
        mp.nhalf = (int)mfma_halves(V);
        mp.half0 = 0;
        q.stats = mp.stats;
        q.nchunks = mp.nhalf;
        const int64_t ntiles = (int64_t)mp.ntiles_v * mp.ntiles_t;
        void *args[] = {&mp};
        if (!launch(lce::mfma_stats_kernel_fn(), (unsigned)(ntiles < cus ? ntiles : cus), 256, args,
                    st))
            return CE_ERR_HIP;
    }
    // forward (library GEMMs): each chunk's logits, then its statistics
    for (int64_t ci = 0; ci < (mfma ? 0 : nch); ++ci) {
        q.v0 = ci * C;
        q.vn = (int)(V - q.v0 < C ? V - q.v0 : C);
        q.chunk_index = (int)ci;
        const void *Wc = (const char *)W + (size_t)q.v0 * D * 2;
        if (!gemm_rm(h, false, true, m, q.vn, d, H, d, Wc, d, 0.0f, Lw, (int)C))
            return CE_ERR_HIP;
        void *args[] = {&q};
        if (!launch(lce::stats_kernel_fn(), row_grid, 256, args, st))
            return CE_ERR_HIP;
    }
    {
        void *args[] = {&q};
        if (!launch(lce::finish_kernel_fn(), row_grid, 256, args, st))
            return CE_ERR_HIP;
    }
    if (reduced) {
        cek::Params p{};
        p.partials = q.partials;
        p.out = out;
        p.out_scale = reduction == CE_MEAN ? 1.0 / (double)M : 1.0;
        unsigned nunits = (unsigned)M;
        void *args[] = {&p, &nunits};
        if (!launch(cek::sum_partials_fn(), 1, 64, args, st))
            return CE_ERR_HIP;
    }
    if (!bwd)
        return CE_OK;

    // backward: recompute each chunk's logits, write its bf16 gradient, then
    // dH (+)= G W_c and dW_c = G^T H
    for (int64_t ci = 0; ci < nch; ++ci) {
        q.v0 = ci * C;
        q.vn = (int)(V - q.v0 < C ? V - q.v0 : C);
        q.chunk_index = (int)ci;
        const void *Wc = (const char *)W + (size_t)q.v0 * D * 2;
        if (mfma) {
            // the chunk's gradient from the matrix-core kernel (persistent)
            mp.v0 = q.v0;
            mp.vn = q.vn;
            mp.ntiles_v = (int)((q.vn + kMfmaTile - 1) / kMfmaTile);
            const int64_t ntiles = (int64_t)mp.ntiles_v * mp.ntiles_t;
            const int cus = cu_count(dev);
            if (cus < 1)
                return CE_ERR_HIP;
            void *args[] = {&mp};
            if (!launch(lce::mfma_grad_kernel_fn(), (unsigned)(ntiles < cus ? ntiles : cus), 256,
                        args, st))
                return CE_ERR_HIP;
            const uint16_t *Gc = mp.G;
            if (!gemm_rm(h, false, false, m, d, q.vn, Gc, (int)C, Wc, d, ci == 0 ? 0.0f : 1.0f, dH,
                         d))
                return CE_ERR_HIP;
            if (!gemm_rm(h, true, false, q.vn, d, m, Gc, (int)C, H, d, 0.0f,
                         dW + (size_t)q.v0 * D, d))
                return CE_ERR_HIP;
            continue;
        }
        if (!gemm_rm(h, false, true, m, q.vn, d, H, d, Wc, d, 0.0f, Lw, (int)C))
            return CE_ERR_HIP;
        void *args[] = {&q};
        if (!launch(lce::grad_kernel_fn(), row_grid, 256, args, st))
            return CE_ERR_HIP;
        if (!gemm_rm(h, false, false, m, d, q.vn, q.G, (int)C, Wc, d, ci == 0 ? 0.0f : 1.0f, dH, d))
            return CE_ERR_HIP;
        if (!gemm_rm(h, true, false, q.vn, d, m, q.G, (int)C, H, d, 0.0f,
                     dW + (size_t)q.v0 * D, d))
            return CE_ERR_HIP;
    }
    return CE_OK;
}

}  // namespace

extern "C" {

int64_t ce_linear_chunk(int64_t M, int64_t D, int64_t V, int64_t chunk)
{
    if (M < 0 || D < 1 || V < 1 || chunk < 0)
        return 0;
    return chunk_for(M, V, chunk);
}

size_t ce_linear_workspace_bytes(int64_t M, int64_t D, int64_t V, int64_t chunk)
{
    if (M < 0 || D < 1 || V < 1 || M > INT_MAX || D > INT_MAX || V > INT_MAX || chunk < 0)
        return 0;
    const int64_t C = chunk_for(M, V, chunk);
    return layout(M, V, C, (V + C - 1) / C).total;
}

int ce_linear_fwd(const void *hidden, const void *weight, const int64_t *targets, int64_t M,
                  int64_t D, int64_t V, ce_reduction_t reduction, float *out, float *lse,
                  int64_t chunk, void *workspace, size_t workspace_bytes, void *stream)
{
    return run(hidden, weight, targets, M, D, V, (int)reduction, out, lse, nullptr, nullptr,
               chunk, workspace, workspace_bytes, stream, false);
}

int ce_linear_fwd_bwd(const void *hidden, const void *weight, const int64_t *targets, int64_t M,
                      int64_t D, int64_t V, ce_reduction_t reduction, float *out, float *lse,
                      float *dhidden, float *dweight, int64_t chunk, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    return run(hidden, weight, targets, M, D, V, (int)reduction, out, lse, dhidden, dweight,
               chunk, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
