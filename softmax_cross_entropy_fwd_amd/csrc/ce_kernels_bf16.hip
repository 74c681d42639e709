// bf16 kernel instances.
#define CE_DT DT_BF16
#define CE_GET_KERNEL get_kernel_bf16
#include "ce_kernels_inst.h"
