// bf16-input MFMA kernel instantiations.
#include "dg_kernels.hpp"
#define DG_TI BF16
#define DG_REGISTER register_mfma_bf16
#include "mfma_inst.inc"
