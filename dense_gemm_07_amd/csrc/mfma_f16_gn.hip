// MFMA kernel instantiations: f16 inputs, load modes LD_GN / LD_GN.
#include "dg_kernels.hpp"
#define DG_TI F16
#define DG_LA LD_GN
#define DG_LB LD_GN
#define DG_ELEMENT_LOADS 1
#define DG_REGISTER register_mfma_f16_gn
#include "mfma_inst.inc"
