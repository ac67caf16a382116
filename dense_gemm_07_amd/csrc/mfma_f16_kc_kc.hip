// MFMA kernel instantiations: f16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_f16_kc_kc(std::vector<KernelEntry> &out) {
    add_shapes<F16, LD_KC, LD_KC>(out);
}
}  // namespace dg
