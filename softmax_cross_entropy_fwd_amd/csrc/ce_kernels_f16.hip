// fp16 kernel instances.
#define CE_DT DT_F16
#define CE_GET_KERNEL get_kernel_f16
#include "ce_kernels_inst.h"
