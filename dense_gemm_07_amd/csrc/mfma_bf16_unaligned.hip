// MFMA kernel instantiations: bf16 inputs.
#include "mfma_units.hpp"
namespace dg {
void register_mfma_bf16_unaligned(std::vector<KernelEntry> &out) {
    add_shapes<BF16, LD_KU, LD_KU>(out);
    add_shapes<BF16, LD_KU, LD_RU>(out);
    add_shapes<BF16, LD_RU, LD_KU>(out);
    add_shapes<BF16, LD_RU, LD_RU>(out);
}
}  // namespace dg
