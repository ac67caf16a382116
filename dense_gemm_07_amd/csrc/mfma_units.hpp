// Registration helpers shared by the MFMA instantiation units.
#pragma once

#include <vector>

#include "dg_kernels.hpp"

namespace dg {

template <int LA, int LB>
constexpr bool direct_to_lds() {
    return (LA == LD_KC || LA == LD_RC) && (LB == LD_KC || LB == LD_RC);
}

// Large tiles with contiguous (but not 16-byte aligned) operands stage them
// through registers into the direct kernel's LDS formats; small tiles and
// element-wise (LD_GN) operands keep the padded-row register kernel (for the
// 64x64 tiles of a 1000x1500x777 product the staged format measured 10 %
// slower: their short steps are bound by per-step costs, not by the LDS
// format).
template <int BM, int BN, int LA, int LB>
constexpr bool staged_direct_format() {
    return BM * BN >= 128 * 128 && (LA == LD_KU || LA == LD_RU) && (LB == LD_KU || LB == LD_RU);
}

template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int S, int EM>
void launch_mode(const GemmArgs &g, hipStream_t s) {
    const unsigned groups = launch_groups(g);
    if constexpr (direct_to_lds<LA, LB>())
        hipLaunchKernelGGL((gemm_mfma_lds<TI, BM, BN, BK, WM, WN, LA, LB, S, EM>), dim3(groups), dim3(WM * WN * 64),
                           0, s, g);
    else if constexpr (staged_direct_format<BM, BN, LA, LB>())
        hipLaunchKernelGGL((gemm_mfma_rs<TI, BM, BN, BK, WM, WN, LA, LB, EM>), dim3(groups), dim3(WM * WN * 64), 0,
                           s, g);
    else
        hipLaunchKernelGGL((gemm_mfma<TI, BM, BN, BK, WM, WN, LA, LB, EM>), dim3(groups), dim3(WM * WN * 64), 0, s, g);
}

// The instantiation for the arguments: split-K partials, fused epilogue, or
// plain stores.
template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int S>
hipError_t launch_mfma(const GemmArgs &g, hipStream_t s) {
    if (g.splits > 1) launch_mode<TI, BM, BN, BK, WM, WN, LA, LB, S, EM_SPLIT>(g, s);
    else if (g.epi) launch_mode<TI, BM, BN, BK, WM, WN, LA, LB, S, EM_FUSED>(g, s);
    else launch_mode<TI, BM, BN, BK, WM, WN, LA, LB, S, EM_STORE>(g, s);
    return hipGetLastError();
}

template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int S>
void add_mfma(std::vector<KernelEntry> &out) {
    out.push_back(KernelEntry{dg_config{BM, BN, BK, 1, WM * WN, S, DG_VARIANT_MFMA, 0, 1}, TI::code, -1, LA, LB,
                              &launch_mfma<TI, BM, BN, BK, WM, WN, LA, LB, S>,
                              direct_to_lds<LA, LB>()                   ? "gemm_mfma_lds"
                              : staged_direct_format<BM, BN, LA, LB>() ? "gemm_mfma_rs"
                                                                         : "gemm_mfma"});
}

// Every tile shape has a two-stage kernel for every load-mode pair (the
// register-staged kernel is two-stage only); the direct-to-LDS kernel adds
// deeper pipelines. Order matters: the heuristic takes the first shape that
// fills the GPU.
template <typename TI, int LA, int LB>
void add_shapes(std::vector<KernelEntry> &out) {
    constexpr bool direct = direct_to_lds<LA, LB>();
    // Element loads (no unit stride) hold eight loads per chunk in flight, and
    // at 256x256x64 that exceeds the register file (the compiler spilled 55
    // registers): those problems use the BK 32 tile instead.
    if constexpr (LA != LD_GN) add_mfma<TI, 256, 256, 64, 2, 4, LA, LB, 2>(out);
    if constexpr (direct) {
        add_mfma<TI, 256, 256, 32, 2, 4, LA, LB, 3>(out);
        add_mfma<TI, 256, 256, 32, 2, 4, LA, LB, 4>(out);
    }
    add_mfma<TI, 256, 256, 32, 2, 4, LA, LB, 2>(out);
    add_mfma<TI, 256, 128, 64, 2, 2, LA, LB, 2>(out);
    add_mfma<TI, 128, 256, 64, 2, 2, LA, LB, 2>(out);
    if constexpr (direct) {
        add_mfma<TI, 128, 128, 64, 2, 2, LA, LB, 3>(out);
        add_mfma<TI, 128, 128, 64, 2, 2, LA, LB, 4>(out);
    }
    add_mfma<TI, 128, 128, 64, 2, 2, LA, LB, 2>(out);
    // small tiles: short K loops are latency-bound, so keep more slices in flight
    if constexpr (direct) {
        add_mfma<TI, 64, 64, 64, 2, 2, LA, LB, 4>(out);
        add_mfma<TI, 64, 64, 32, 2, 2, LA, LB, 8>(out);
    }
    add_mfma<TI, 64, 64, 64, 2, 2, LA, LB, 2>(out);
    add_mfma<TI, 64, 64, 32, 2, 2, LA, LB, 2>(out);
}

}  // namespace dg
