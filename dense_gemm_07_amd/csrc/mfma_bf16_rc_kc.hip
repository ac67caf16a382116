// MFMA kernel instantiations: bf16 inputs, load modes LD_RC / LD_KC.
#include "dg_kernels.hpp"
#define DG_TI BF16
#define DG_LA LD_RC
#define DG_LB LD_KC
#define DG_ELEMENT_LOADS 0
#define DG_REGISTER register_mfma_bf16_rc_kc
#include "mfma_inst.inc"
