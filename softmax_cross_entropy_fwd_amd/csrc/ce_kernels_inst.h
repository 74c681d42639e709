// ce_kernels_inst.h -- instantiates every kernel shape for one storage type.
// Included once per type with CE_DT and CE_GET_KERNEL defined.
#include "ce_device.h"
#include "ce_internal.h"

namespace cek {
namespace {

template <int DT, bool BWD>
KernelRef pick(int kind, int a, int b)
{
#define CE_ROWS(G, K) \
    if (a == G && b == K) return KernelRef{(const void *)&rows_kernel<DT, G, K, BWD>, 256};
#define CE_WG(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&wg_kernel<DT, W, K, BWD>, W * 64};
#define CE_STREAM(W, K) \
    if (a == W && b == K) return KernelRef{(const void *)&stream_kernel<DT, W, K, BWD>, W * 64};
    if (kind == KIND_ROWS) {
        CE_ROWS(1, 1) CE_ROWS(1, 2) CE_ROWS(1, 4) CE_ROWS(2, 4) CE_ROWS(4, 4) CE_ROWS(8, 4)
        CE_ROWS(16, 4) CE_ROWS(32, 4) CE_ROWS(64, 4) CE_ROWS(64, 8) CE_ROWS(64, 16)
        CE_ROWS(4, 8) CE_ROWS(8, 2) CE_ROWS(16, 2) CE_ROWS(32, 1) CE_ROWS(32, 8) CE_ROWS(32, 16)
    } else if (kind == KIND_WG) {
        CE_WG(4, 8) CE_WG(8, 8) CE_WG(8, 12) CE_WG(8, 16) CE_WG(16, 8) CE_WG(16, 12) CE_WG(16, 16)
        CE_WG(4, 16) CE_WG(16, 4)
    } else if (kind == KIND_STREAM) {
        CE_STREAM(4, 8) CE_STREAM(8, 4) CE_STREAM(8, 8) CE_STREAM(16, 4) CE_STREAM(4, 16)
    }
#undef CE_ROWS
#undef CE_WG
#undef CE_STREAM
    return KernelRef{nullptr, 0};
}

}  // namespace

KernelRef CE_GET_KERNEL(int kind, int a, int b, bool bwd)
{
    return bwd ? pick<CE_DT, true>(kind, a, b) : pick<CE_DT, false>(kind, a, b);
}

}  // namespace cek
