// MFMA kernel instantiations: f16 inputs, load modes LD_RC / LD_RC.
#include "dg_kernels.hpp"
#define DG_TI F16
#define DG_LA LD_RC
#define DG_LB LD_RC
#define DG_ELEMENT_LOADS 0
#define DG_REGISTER register_mfma_f16_rc_rc
#include "mfma_inst.inc"
