// ce_kernels_inst.h -- instantiates every kernel shape for one storage type.
// Included once per type with CE_DT and CE_GET_KERNEL defined.
#include "ce_device.h"
#include "ce_internal.h"

namespace cek {
namespace {

template <int DT, bool BWD, bool EXACT>
KernelRef pick(int kind, int a, int b, int nbuf)
{
#define CE_ROWS(G, K)                                                                           \
    if (a == G && b == K)                                                                       \
        return nbuf == 2 ? KernelRef{(const void *)&rows_kernel<DT, G, K, BWD, EXACT, 2>, 256}  \
                         : KernelRef{(const void *)&rows_kernel<DT, G, K, BWD, EXACT, 1>, 256};
#define CE_WG(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&wg_kernel<DT, W, K, BWD, EXACT>, W * 64};
#define CE_STREAM(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&stream_kernel<DT, W, K, BWD>, W * 64};
    if (kind == KIND_ROWS && nbuf >= 16) {   // 16-wave workgroups (nbuf = 16 + buffers)
        if (a == 64 && b == 16)
            return nbuf == 17 ? KernelRef{(const void *)&rows_kernel<DT, 64, 16, BWD, EXACT, 1, 16>, 1024}
                              : KernelRef{(const void *)&rows_kernel<DT, 64, 16, BWD, EXACT, 2, 16>, 1024};
        if (a == 4 && b == 8)
            return nbuf == 17 ? KernelRef{(const void *)&rows_kernel<DT, 4, 8, BWD, EXACT, 1, 16>, 1024}
                              : KernelRef{(const void *)&rows_kernel<DT, 4, 8, BWD, EXACT, 2, 16>, 1024};
    } else if (kind == KIND_ROWS) {
        CE_ROWS(1, 1) CE_ROWS(1, 2) CE_ROWS(1, 4) CE_ROWS(2, 4) CE_ROWS(4, 4) CE_ROWS(8, 4)
        CE_ROWS(16, 4) CE_ROWS(32, 4) CE_ROWS(64, 4) CE_ROWS(64, 8) CE_ROWS(64, 16)
        CE_ROWS(4, 8) CE_ROWS(8, 2) CE_ROWS(16, 2) CE_ROWS(32, 1) CE_ROWS(32, 8) CE_ROWS(32, 16)
        CE_ROWS(32, 32) CE_ROWS(2, 16)
    } else if (kind == KIND_WG) {
        CE_WG(4, 8) CE_WG(8, 8) CE_WG(8, 12) CE_WG(8, 16) CE_WG(16, 8) CE_WG(16, 12) CE_WG(16, 16)
        CE_WG(4, 16) CE_WG(16, 4)
    } else if (kind == KIND_WSTREAM && !EXACT && !BWD) {
        if (a == 1 && b == 4) return KernelRef{(const void *)&wstream_kernel<DT, 4>, 256};
        if (a == 1 && b == 2) return KernelRef{(const void *)&wstream_kernel<DT, 2>, 256};
        if (a == 1 && b == 8) return KernelRef{(const void *)&wstream_kernel<DT, 8>, 256};
    } else if (kind == KIND_STREAM && !EXACT) {
        CE_STREAM(4, 8) CE_STREAM(8, 4) CE_STREAM(8, 8) CE_STREAM(16, 4) CE_STREAM(4, 16)
        CE_STREAM(1, 4) CE_STREAM(2, 4) CE_STREAM(4, 4) CE_STREAM(1, 8) CE_STREAM(2, 8)
        CE_STREAM(1, 16) CE_STREAM(16, 2) CE_STREAM(16, 1) CE_STREAM(8, 2)
    }
#undef CE_ROWS
#undef CE_WG
#undef CE_STREAM
    return KernelRef{nullptr, 0};
}

}  // namespace

KernelRef CE_GET_KERNEL(int kind, int a, int b, bool bwd, bool exact, int nbuf)
{
    if (exact)
        return bwd ? pick<CE_DT, true, true>(kind, a, b, nbuf)
                   : pick<CE_DT, false, true>(kind, a, b, nbuf);
    return bwd ? pick<CE_DT, true, false>(kind, a, b, nbuf)
               : pick<CE_DT, false, false>(kind, a, b, nbuf);
}

}  // namespace cek
