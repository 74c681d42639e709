// bf16 kernel instances: epilogue (fused backward, softmax, log-softmax, backward from saved lse).
#define CE_DT DT_BF16
#define CE_PART 1
#define CE_GET_KERNEL get_kernel_bf16_epi
#include "ce_kernels_inst.h"
