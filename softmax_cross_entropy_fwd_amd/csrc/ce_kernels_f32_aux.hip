// f32 kernel instances: softmax, log-softmax, backward from a given log-sum-exp; the split-row kernels.
#define CE_DT DT_F32
#define CE_PART 2
#define CE_GET_KERNEL get_kernel_f32_aux
#define CE_SPLIT_KERNELS split_kernels_f32
#include "ce_kernels_inst.h"
