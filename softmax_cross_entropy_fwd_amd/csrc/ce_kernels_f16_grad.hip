// f16 kernel instances: fused forward + in-place backward.
#define CE_DT DT_F16
#define CE_PART 1
#define CE_GET_KERNEL get_kernel_f16_grad
#include "ce_kernels_inst.h"
