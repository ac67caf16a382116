// MFMA kernel instantiations: bf16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_bf16_gn(std::vector<KernelEntry> &out) {
    add_shapes<BF16, LD_GN, LD_GN>(out);
}
}  // namespace dg
