// MFMA kernel instantiations: f16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_f16_gn(std::vector<KernelEntry> &out) {
    add_shapes<F16, LD_GN, LD_GN>(out);
}
}  // namespace dg
