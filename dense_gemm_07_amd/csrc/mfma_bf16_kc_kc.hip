// MFMA kernel instantiations: bf16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_bf16_kc_kc(std::vector<KernelEntry> &out) {
    add_shapes<BF16, LD_KC, LD_KC>(out);
}
}  // namespace dg
