// bf16 kernel instances: forward.
#define CE_DT DT_BF16
#define CE_PART 0
#define CE_GET_KERNEL get_kernel_bf16_fwd
#include "ce_kernels_inst.h"
