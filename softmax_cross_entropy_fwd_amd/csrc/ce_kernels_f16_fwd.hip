// f16 kernel instances: forward.
#define CE_DT DT_F16
#define CE_PART 0
#define CE_GET_KERNEL get_kernel_f16_fwd
#include "ce_kernels_inst.h"
