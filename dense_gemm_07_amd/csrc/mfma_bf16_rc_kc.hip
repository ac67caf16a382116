// MFMA kernel instantiations: bf16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_bf16_rc_kc(std::vector<KernelEntry> &out) {
    add_shapes<BF16, LD_RC, LD_KC>(out);
}
}  // namespace dg
