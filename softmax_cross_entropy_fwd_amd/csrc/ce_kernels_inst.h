// ce_kernels_inst.h -- instantiates the kernel shapes for one storage type and
// one group of operations.  Included by the per-type units with CE_DT, CE_PART
// (0: forward, 1: fused backward, 2: softmax, log-softmax and the backward
// from a given log-sum-exp) and CE_GET_KERNEL defined.
#include "ce_device.h"
#include "ce_internal.h"

namespace cek {
namespace {

#define CE_ROWS(G, K)                                                                            \
    if (a == G && b == K)                                                                        \
        return nbuf == 2 ? KernelRef{(const void *)&rows_kernel<DT, G, K, OP, EXACT, 2>, 256}    \
                         : KernelRef{(const void *)&rows_kernel<DT, G, K, OP, EXACT, 1>, 256};
#define CE_ROWS1(G, K) \
    if (a == G && b == K) return KernelRef{(const void *)&rows_kernel<DT, G, K, OP, EXACT, 1>, 256};
#define CE_WG(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&wg_kernel<DT, W, K, OP, EXACT>, W * 64};
// 8-wave workgroups held to 128 VGPRs, so that two share a CU
#define CE_WG2(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&wg_kernel<DT, W, K, OP, EXACT, 4>, W * 64};
#define CE_STREAM(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&stream_kernel<DT, W, K, OP>, W * 64};

// Every shape, for the forward and the fused in-place backward.
template <int DT, int OP, bool EXACT>
KernelRef pick_all(int kind, int a, int b, int nbuf)
{
    if (kind == KIND_ROWS && nbuf >= 16) {   // 16-wave workgroups (nbuf = 16 + buffers)
        if (a == 64 && b == 16)
            return nbuf == 17 ? KernelRef{(const void *)&rows_kernel<DT, 64, 16, OP, EXACT, 1, 16>, 1024}
                              : KernelRef{(const void *)&rows_kernel<DT, 64, 16, OP, EXACT, 2, 16>, 1024};
        if (a == 4 && b == 8)
            return nbuf == 17 ? KernelRef{(const void *)&rows_kernel<DT, 4, 8, OP, EXACT, 1, 16>, 1024}
                              : KernelRef{(const void *)&rows_kernel<DT, 4, 8, OP, EXACT, 2, 16>, 1024};
    } else if (kind == KIND_ROWS) {
        CE_ROWS(1, 1) CE_ROWS(1, 2) CE_ROWS(1, 4) CE_ROWS(2, 4) CE_ROWS(4, 4) CE_ROWS(8, 4)
        CE_ROWS(16, 4) CE_ROWS(32, 4) CE_ROWS(64, 4) CE_ROWS(64, 8) CE_ROWS(64, 16)
        CE_ROWS(4, 8) CE_ROWS(8, 2) CE_ROWS(16, 2) CE_ROWS(32, 1) CE_ROWS(32, 8) CE_ROWS(32, 16)
        CE_ROWS(32, 32) CE_ROWS(2, 16)
        // 5 or 6 vectors per lane: rows just over a tile size
        CE_ROWS1(8, 5) CE_ROWS1(8, 6) CE_ROWS1(16, 5) CE_ROWS1(16, 6) CE_ROWS1(32, 5)
        CE_ROWS1(32, 6)
    } else if (kind == KIND_WG) {
        CE_WG(4, 8) CE_WG(8, 8) CE_WG(8, 12) CE_WG(8, 16) CE_WG(16, 8) CE_WG(16, 12) CE_WG(16, 16)
        CE_WG(4, 16) CE_WG(16, 4) CE_WG(16, 2) CE_WG(16, 3) CE_WG(16, 5) CE_WG(16, 6) CE_WG(16, 7)
    } else if (kind == KIND_WG2 && DT != DT_F32) {
        CE_WG2(8, 9) CE_WG2(8, 10) CE_WG2(8, 11) CE_WG2(8, 12) CE_WG2(8, 13)
    } else if (kind == KIND_WSTREAM && !EXACT && OP == EPI_NONE) {
        if (a == 1 && b == 4) return KernelRef{(const void *)&wstream_kernel<DT, 4>, 256};
        if (a == 1 && b == 2) return KernelRef{(const void *)&wstream_kernel<DT, 2>, 256};
        if (a == 1 && b == 8) return KernelRef{(const void *)&wstream_kernel<DT, 8>, 256};
    } else if (kind == KIND_STREAM && !EXACT) {
        CE_STREAM(4, 8) CE_STREAM(8, 4) CE_STREAM(8, 8) CE_STREAM(16, 4) CE_STREAM(4, 16)
        CE_STREAM(1, 4) CE_STREAM(2, 4) CE_STREAM(4, 4) CE_STREAM(1, 8) CE_STREAM(2, 8)
        CE_STREAM(1, 16) CE_STREAM(16, 2) CE_STREAM(16, 1) CE_STREAM(8, 2)
    }
    return KernelRef{nullptr, 0};
}

// The shapes the plan table uses, for softmax, log-softmax and the backward
// from a given log-sum-exp.
template <int DT, int OP, bool EXACT>
KernelRef pick_table(int kind, int a, int b, int nbuf)
{
    if (kind == KIND_ROWS) {
        if (a == 4 && b == 8)
            return nbuf == 2 ? KernelRef{(const void *)&rows_kernel<DT, 4, 8, OP, EXACT, 2>, 256}
                             : KernelRef{(const void *)&rows_kernel<DT, 4, 8, OP, EXACT, 1>, 256};
        CE_ROWS1(1, 1) CE_ROWS1(1, 2) CE_ROWS1(1, 4) CE_ROWS1(2, 4) CE_ROWS1(4, 4)
        CE_ROWS1(16, 4) CE_ROWS1(32, 4) CE_ROWS1(64, 4) CE_ROWS1(64, 8) CE_ROWS1(64, 16)
        CE_ROWS1(8, 5) CE_ROWS1(8, 6) CE_ROWS1(16, 5) CE_ROWS1(16, 6) CE_ROWS1(32, 5)
        CE_ROWS1(32, 6)
    } else if (kind == KIND_WG) {
        CE_WG(16, 2) CE_WG(16, 3) CE_WG(16, 4) CE_WG(16, 5) CE_WG(16, 6) CE_WG(16, 7)
        CE_WG(16, 8) CE_WG(16, 12) CE_WG(16, 16)
    } else if (kind == KIND_WG2 && DT != DT_F32) {
        CE_WG2(8, 9) CE_WG2(8, 10) CE_WG2(8, 11) CE_WG2(8, 12) CE_WG2(8, 13)
    } else if (kind == KIND_STREAM && !EXACT) {
        CE_STREAM(4, 4) CE_STREAM(8, 4) CE_STREAM(16, 4)
    }
    return KernelRef{nullptr, 0};
}

#undef CE_ROWS
#undef CE_ROWS1
#undef CE_WG
#undef CE_WG2
#undef CE_STREAM

}  // namespace

KernelRef CE_GET_KERNEL(int op, int kind, int a, int b, bool exact, int nbuf)
{
#if CE_PART == 0
    if (op == EPI_NONE)
        return exact ? pick_all<CE_DT, EPI_NONE, true>(kind, a, b, nbuf)
                     : pick_all<CE_DT, EPI_NONE, false>(kind, a, b, nbuf);
#elif CE_PART == 1
    if (op == EPI_GRAD)
        return exact ? pick_all<CE_DT, EPI_GRAD, true>(kind, a, b, nbuf)
                     : pick_all<CE_DT, EPI_GRAD, false>(kind, a, b, nbuf);
#else
    if (op == EPI_SOFTMAX)
        return exact ? pick_table<CE_DT, EPI_SOFTMAX, true>(kind, a, b, nbuf)
                     : pick_table<CE_DT, EPI_SOFTMAX, false>(kind, a, b, nbuf);
    if (op == EPI_LOGSOFTMAX)
        return exact ? pick_table<CE_DT, EPI_LOGSOFTMAX, true>(kind, a, b, nbuf)
                     : pick_table<CE_DT, EPI_LOGSOFTMAX, false>(kind, a, b, nbuf);
    if (op == EPI_LSE_GRAD)
        return exact ? pick_table<CE_DT, EPI_LSE_GRAD, true>(kind, a, b, nbuf)
                     : pick_table<CE_DT, EPI_LSE_GRAD, false>(kind, a, b, nbuf);
#endif
    return KernelRef{nullptr, 0};
}

#if CE_PART == 2
SplitKernels CE_SPLIT_KERNELS()
{
    static_assert(kSplitChunk == 4 * 64 * 4, "chunk = W x 64 x K of the split kernels");
    SplitKernels s;
    s.stats = (const void *)&split_stats_kernel<CE_DT, 4, 4>;
    s.finish = (const void *)&split_epi_kernel<CE_DT, 1, 1, EPI_NONE>;
    s.epi[EPI_NONE] = nullptr;
    s.epi[EPI_GRAD] = (const void *)&split_epi_kernel<CE_DT, 4, 4, EPI_GRAD>;
    s.epi[EPI_SOFTMAX] = (const void *)&split_epi_kernel<CE_DT, 4, 4, EPI_SOFTMAX>;
    s.epi[EPI_LOGSOFTMAX] = (const void *)&split_epi_kernel<CE_DT, 4, 4, EPI_LOGSOFTMAX>;
    s.epi[EPI_LSE_GRAD] = (const void *)&split_epi_kernel<CE_DT, 4, 4, EPI_LSE_GRAD>;
    s.fix = (const void *)&split_fix_kernel<CE_DT>;
    return s;
}
#endif

}  // namespace cek
