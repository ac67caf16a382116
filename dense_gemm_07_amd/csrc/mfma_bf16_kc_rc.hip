// MFMA kernel instantiations: bf16 inputs, load modes LD_KC / LD_RC.
#include "dg_kernels.hpp"
#define DG_TI BF16
#define DG_LA LD_KC
#define DG_LB LD_RC
#define DG_ELEMENT_LOADS 0
#define DG_REGISTER register_mfma_bf16_kc_rc
#include "mfma_inst.inc"
