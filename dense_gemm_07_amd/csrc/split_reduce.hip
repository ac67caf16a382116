// Instantiations of the split-K reduction kernel, one per MFMA tile shape and
// wave layout (the layouts the MFMA units compile: 8 waves as 2 x 4, 4 waves
// as 2 x 2).
#include "dg_kernels.hpp"

namespace dg {

template <int BM, int BN, int WM, int WN>
static hipError_t launch_reduce(const GemmArgs &g, hipStream_t s) {
    const unsigned groups = (unsigned)g.grid_m * (unsigned)g.grid_n * (unsigned)g.batch;
    hipLaunchKernelGGL((gemm_split_reduce<BM, BN, WM, WN>), dim3(groups), dim3(WM * WN * 64), 0, s, g);
    return hipGetLastError();
}

LaunchFn split_reduce_kernel(int block_m, int block_n, int waves) {
    if (waves == 8 && block_m == 256 && block_n == 256) return &launch_reduce<256, 256, 2, 4>;
    if (waves == 4 && block_m == 256 && block_n == 128) return &launch_reduce<256, 128, 2, 2>;
    if (waves == 4 && block_m == 128 && block_n == 256) return &launch_reduce<128, 256, 2, 2>;
    if (waves == 4 && block_m == 128 && block_n == 128) return &launch_reduce<128, 128, 2, 2>;
    if (waves == 4 && block_m == 64 && block_n == 64) return &launch_reduce<64, 64, 2, 2>;
    return nullptr;
}

}  // namespace dg
