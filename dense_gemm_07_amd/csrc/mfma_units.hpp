// Registration helpers shared by the MFMA instantiation units.
#pragma once

#include <vector>

#include "dg_kernels.hpp"

namespace dg {

template <int LA, int LB>
constexpr bool direct_to_lds() {
    return (LA == LD_KC || LA == LD_RC) && (LB == LD_KC || LB == LD_RC);
}

// Contiguous (but not 16-byte aligned) operands are staged through registers
// into the direct kernel's LDS formats on large tiles, and on small tiles
// when one operand is row-contiguous; small tiles with both operands
// k-contiguous, and element-wise (LD_GN) operands, keep the padded-row
// register kernel. Measured on MI355X: for the 64x64 tiles of a
// 1000x1500x777 product with k-contiguous operands the staged format is 10 %
// slower (short steps bound by per-step costs); with a row-contiguous B
// (1000x1500x2048, B row-major) the padded-row kernel's 8x8 register
// transposes, done by every thread of a 256-thread tile for 64 blocks, made
// it 5x slower than the staged format.
template <int BM, int BN, int LA, int LB>
constexpr bool staged_direct_format() {
    return (BM * BN >= 128 * 128 || LA == LD_RU || LB == LD_RU) && (LA == LD_KU || LA == LD_RU) &&
           (LB == LD_KU || LB == LD_RU);
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

// Tile shapes that are also compiled as stream-K kernels: the 64x64 tile the
// heuristic takes for small problems and the 128x128 tile, at BK 64 (for the
// register-staged kernel, whose pipeline depth is fixed, the two-stage entry;
// for the direct kernel, the 64x64 tile's four stages), on the direct and the
// padded-row register kernels. Not the 256x256 tile (with the piece loop
// around it, its eight waves' registers overflow: the compiler spilled inside
// the K loop), nor the staged kernel (the same, at 256x256).
template <int BM, int BN, int BK, int S, int LA, int LB>
constexpr bool has_stream_k() {
    if (BK != 64 || staged_direct_format<BM, BN, LA, LB>()) return false;
    if (BM == 64 && BN == 64) return direct_to_lds<LA, LB>() ? S == 4 : S == 2;
    return BM == 128 && BN == 128 && S == 2;
}

// The instantiation for the arguments: stream-K, split-K partials, fused
// epilogue, or plain stores.
template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int S>
hipError_t launch_mfma(const GemmArgs &g, hipStream_t s) {
    if constexpr (has_stream_k<BM, BN, BK, S, LA, LB>())
        if (g.sk_groups > 0) {
            launch_mode<TI, BM, BN, BK, WM, WN, LA, LB, S, EM_STREAMK>(g, s);
            return hipGetLastError();
        }
    if (g.sk_groups > 0) return hipErrorInvalidValue;  // the host checks KernelEntry::stream_k first
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
                                                                         : "gemm_mfma",
                              has_stream_k<BM, BN, BK, S, LA, LB>()});
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
