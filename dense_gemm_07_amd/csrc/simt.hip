// Instantiations of the scalar-FMA kernel: every (input, output) dtype pair.
#include "dg_kernels.hpp"

namespace dg {

template <typename TI, typename TO, int BM, int BN, int BK>
static hipError_t launch_simt(const GemmArgs &g, hipStream_t s) {
    hipLaunchKernelGGL((gemm_simt<TI, TO, BM, BN, BK>), dim3(launch_groups(g)), dim3(256), 0, s, g);
    return hipGetLastError();
}

#define DG_SIMT(TI, TO, BM, BN, BK)                                                          \
    out.push_back(KernelEntry{dg_config{BM, BN, BK, 1, 4, 1, DG_VARIANT_SIMT, 0, 1}, TI::code,  \
                              TO::code, -1, -1, &launch_simt<TI, TO, BM, BN, BK>,            \
                              "simt_" #TI "_" #TO "_" #BM "x" #BN "x" #BK})
#define DG_SIMT_TILES(TI, TO) \
    DG_SIMT(TI, TO, 64, 64, 16); \
    DG_SIMT(TI, TO, 32, 32, 16)

void register_simt(std::vector<KernelEntry> &out) {
    DG_SIMT_TILES(F32, F32);
    DG_SIMT_TILES(F32, F16);
    DG_SIMT_TILES(F32, BF16);
    DG_SIMT_TILES(F16, F32);
    DG_SIMT_TILES(F16, F16);
    DG_SIMT_TILES(F16, BF16);
    DG_SIMT_TILES(BF16, F32);
    DG_SIMT_TILES(BF16, F16);
    DG_SIMT_TILES(BF16, BF16);
}

}  // namespace dg
