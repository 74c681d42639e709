// f16 kernel instances: softmax, log-softmax, backward from a given log-sum-exp.
#define CE_DT DT_F16
#define CE_PART 2
#define CE_GET_KERNEL get_kernel_f16_aux
#include "ce_kernels_inst.h"
