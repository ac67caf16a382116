// fp32-input matrix-core kernel instantiations (v_mfma_f32_32x32x2_f32): every
// load-mode pair, plain / fused-epilogue / split-K instantiations.
#include "dg_kernels.hpp"

namespace dg {

template <int BM, int BN, int BK, int LA, int LB>
static hipError_t launch_mfma_f32(const GemmArgs &g, hipStream_t s) {
    if (g.sk_groups > 0) return hipErrorInvalidValue;  // no stream-K instantiation (the host checks first)
    const dim3 grid(launch_groups(g)), block(256);
    if (g.splits > 1) hipLaunchKernelGGL((gemm_mfma_f32<BM, BN, BK, 2, 2, LA, LB, EM_SPLIT>), grid, block, 0, s, g);
    else if (g.epi) hipLaunchKernelGGL((gemm_mfma_f32<BM, BN, BK, 2, 2, LA, LB, EM_FUSED>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((gemm_mfma_f32<BM, BN, BK, 2, 2, LA, LB, EM_STORE>), grid, block, 0, s, g);
    return hipGetLastError();
}

template <int LA, int LB>
static void add_f32(std::vector<KernelEntry> &out) {
    out.push_back(KernelEntry{dg_config{128, 128, 32, 1, 4, 2, DG_VARIANT_MFMA, 0, 1}, DG_F32, -1, LA, LB,
                              &launch_mfma_f32<128, 128, 32, LA, LB>, "gemm_mfma_f32", false});
    out.push_back(KernelEntry{dg_config{64, 64, 32, 1, 4, 2, DG_VARIANT_MFMA, 0, 1}, DG_F32, -1, LA, LB,
                              &launch_mfma_f32<64, 64, 32, LA, LB>, "gemm_mfma_f32", false});
}

void register_mfma_f32(std::vector<KernelEntry> &out) {
    add_f32<LD_KC, LD_KC>(out);
    add_f32<LD_KC, LD_RC>(out);
    add_f32<LD_KC, LD_GN>(out);
    add_f32<LD_RC, LD_KC>(out);
    add_f32<LD_RC, LD_RC>(out);
    add_f32<LD_RC, LD_GN>(out);
    add_f32<LD_GN, LD_KC>(out);
    add_f32<LD_GN, LD_RC>(out);
    add_f32<LD_GN, LD_GN>(out);
}

}  // namespace dg
