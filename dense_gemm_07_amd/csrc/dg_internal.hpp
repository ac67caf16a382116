// Internal types shared by the host dispatcher and the kernel translation
// units of the dense GEMM library. Not part of the C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "dg.h"

namespace dg {

// Runtime arguments of one launch. Sizes fit in int32 (checked on the host);
// strides are element strides (int64: a leading dimension times a row index
// can pass 2^31).
struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    int32_t M, N, K;
    int32_t grid_m, grid_n;
    int32_t group_m;
    int32_t xcd_remap;
    int32_t num_xcd;
    int32_t out_dtype;  // dg_dtype of C (the MFMA kernels pick the store at run time)
    int64_t sam, sak, sbk, sbn, scm, scn;
};

// How an operand tile is fetched from global memory. The operand is viewed
// as rows x K (rows = M for A, N for B) with a row stride and a k stride.
// LD_KC / LD_RC select the direct-to-LDS kernel; LD_KU / LD_RU / LD_GN the
// register-staged kernel.
enum LoadMode : int32_t {
    LD_KC = 0,  // k-contiguous (k stride 1), 16-byte aligned rows, K % 8 == 0
    LD_RC = 1,  // row-contiguous (row stride 1), 16-byte aligned k-lines, rows % 8 == 0
    LD_GN = 2,  // anything else: element loads through both strides
    LD_KU = 3,  // k-contiguous, any element alignment
    LD_RU = 4,  // row-contiguous, any element alignment
};

using LaunchFn = hipError_t (*)(const GemmArgs &, hipStream_t);

// One compiled kernel instantiation.
struct KernelEntry {
    dg_config cfg;      // block sizes, waves, stages, variant (group_m / xcd_remap unused)
    int32_t in_dtype;   // dg_dtype of A and B
    int32_t out_dtype;  // dg_dtype of C, or -1 if the kernel handles every output dtype
    int32_t load_a;     // LoadMode for A (-1: any, the kernel uses element loads)
    int32_t load_b;     // LoadMode for B (-1: any)
    LaunchFn launch;
    const char *name;
};

// Registration hooks, one per kernel translation unit.
void register_simt(std::vector<KernelEntry> &out);
#define DG_DECLARE_MFMA_HOOKS(t)                               \
    void register_mfma_##t##_kc_rc(std::vector<KernelEntry> &out); \
    void register_mfma_##t##_kc_kc(std::vector<KernelEntry> &out); \
    void register_mfma_##t##_rc_rc(std::vector<KernelEntry> &out); \
    void register_mfma_##t##_rc_kc(std::vector<KernelEntry> &out); \
    void register_mfma_##t##_gn(std::vector<KernelEntry> &out);    \
    void register_mfma_##t##_unaligned(std::vector<KernelEntry> &out);
DG_DECLARE_MFMA_HOOKS(bf16)
DG_DECLARE_MFMA_HOOKS(f16)
#undef DG_DECLARE_MFMA_HOOKS

// ---------------------------------------------------------------------------
// Tile launch order. A workgroup id is mapped to the C tile it computes:
//  1. XCD-aware renumbering (optional). Workgroups are handed to the XCDs
//     round-robin (wg % num_xcd), and each XCD has its own L2. The ids that
//     land on one XCD are given consecutive logical numbers, so the tiles
//     one L2 serves are neighbours in the order of step 2.
//  2. Group-major order over the logical number ("I Wrote a GPU Matmul Kernel
//     From Scratch in Triton", Step 4): groups of group_m tile rows are walked
//     column by column, so consecutive ids cover a compact block of C and
//     share rows of A and columns of B. group_m = 1 is plain row-major order
//     (the 1D decode of "Triton：04 Matmul、Autotune 与 PyTorch 集成").
// Both steps are bijections on [0, grid_m * grid_n).
// ---------------------------------------------------------------------------
__host__ __device__ inline void tile_coords(int wg, int grid_m, int grid_n, int group_m,
                                            int xcd_remap, int num_xcd, int &pid_m, int &pid_n) {
    const int tiles = grid_m * grid_n;
    int lid = wg;
    if (xcd_remap && num_xcd > 1) {
        const int x = wg % num_xcd;       // XCD this id is dispatched to
        const int local = wg / num_xcd;   // its rank among that XCD's ids
        const int q = tiles / num_xcd, r = tiles % num_xcd;
        // XCDs 0..r-1 receive q+1 ids, the others q.
        lid = x * q + (x < r ? x : r) + local;
    }
    const int g = group_m < 1 ? 1 : group_m;
    const int per_group = g * grid_n;
    const int group_id = lid / per_group;
    const int first_m = group_id * g;
    const int rows_here = (grid_m - first_m) < g ? (grid_m - first_m) : g;
    const int in_group = lid - group_id * per_group;
    pid_m = first_m + in_group % rows_here;
    pid_n = in_group / rows_here;
}

}  // namespace dg
