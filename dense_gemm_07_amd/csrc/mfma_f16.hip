// fp16-input MFMA kernel instantiations.
#include "dg_kernels.hpp"
#define DG_TI F16
#define DG_REGISTER register_mfma_f16
#include "mfma_inst.inc"
