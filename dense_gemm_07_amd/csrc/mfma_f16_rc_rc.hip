// MFMA kernel instantiations: f16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_f16_rc_rc(std::vector<KernelEntry> &out) {
    add_shapes<F16, LD_RC, LD_RC>(out);
}
}  // namespace dg
