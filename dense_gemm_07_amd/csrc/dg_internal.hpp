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
//
// One launch covers `batch` products of the same shape (product b reads
// A + b*bsa, B + b*bsb, R + b*bsr, bias + b*bsbias and writes C + b*bsc) and
// `splits` K ranges per output tile: range s covers k in
// [s*k_chunk, min(K, (s+1)*k_chunk)). Workgroup ids enumerate
// (product, range, tile) with the tile fastest.
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
    // batch and split-K
    int32_t batch;          // products in this launch, >= 1
    int32_t splits;         // K ranges per tile, >= 1; > 1 only for the MFMA kernels
    int32_t k_chunk;        // K elements per range (a multiple of block_k when splits > 1)
    int64_t bsa, bsb, bsc;  // batch strides of A, B, C
    float *ws;              // split-K partial tiles (fp32); stream-K flags and partials
    // fused epilogue: C = act(alpha * acc + beta * R + bias)
    int32_t epi;            // 0: C = acc (the other fields are unused); 1: the general form
    int32_t act;            // dg_activation
    float alpha, beta;      // beta == 0: R is not read
    const void *R;          // residual (C itself for an in-place beta * C)
    int64_t srm, srn, bsr;
    int32_t r_dtype;
    int32_t bias_dtype;
    const void *bias;       // NULL: no bias
    int64_t sbias, bsbias;
    int32_t bias_per_row;   // 0: bias[j], one per column; 1: bias[i], one per row
    // stream-K (EM_STREAMK kernels)
    int32_t sk_groups;      // > 0: stream-K over this many workgroups (ranks); 0: one workgroup per work item
    int32_t sk_tiles;       // tiles whose K steps are shared out; the rest are whole-tile work
    int32_t sk_iters;       // K steps per tile, ceil(K / block_k)
    int32_t sk_base;        // S / sk_groups, S = sk_tiles * sk_iters < 2^31
    int32_t sk_extra;       // S % sk_groups: ranks below it take one step more
    uint32_t sk_epoch;      // this launch's flag value (never 0)
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
    bool stream_k;      // also compiled as a stream-K kernel (k_splits = DG_STREAM_K)
};

// Registration hooks, one per kernel translation unit.
void register_simt(std::vector<KernelEntry> &out);
void register_mfma_f32(std::vector<KernelEntry> &out);
// The split-K reduction kernel for an MFMA tile shape (nullptr if none).
LaunchFn split_reduce_kernel(int block_m, int block_n, int waves);
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

// Step 1 over `total` workgroup ids.
__host__ __device__ inline int xcd_rank(int wg, int total, int num_xcd) {
    const int x = wg % num_xcd;       // XCD this id is dispatched to
    const int local = wg / num_xcd;   // its rank among that XCD's ids
    const int q = total / num_xcd, r = total % num_xcd;
    // XCDs 0..r-1 receive q+1 ids, the others q.
    return x * q + (x < r ? x : r) + local;
}

// Step 2: logical tile number -> (pid_m, pid_n).
__host__ __device__ inline void group_major(int lid, int grid_m, int grid_n, int group_m, int &pid_m, int &pid_n) {
    const int g = group_m < 1 ? 1 : group_m;
    const int per_group = g * grid_n;
    const int group_id = lid / per_group;
    const int first_m = group_id * g;
    const int rows_here = (grid_m - first_m) < g ? (grid_m - first_m) : g;
    const int in_group = lid - group_id * per_group;
    pid_m = first_m + in_group % rows_here;
    pid_n = in_group / rows_here;
}

__host__ __device__ inline void tile_coords(int wg, int grid_m, int grid_n, int group_m,
                                            int xcd_remap, int num_xcd, int &pid_m, int &pid_n) {
    const int tiles = grid_m * grid_n;
    const int lid = (xcd_remap && num_xcd > 1) ? xcd_rank(wg, tiles, num_xcd) : wg;
    group_major(lid, grid_m, grid_n, group_m, pid_m, pid_n);
}

// What one workgroup of a launch computes: tile (pm, pn) of product `prod`,
// K range `split`; `slot` = prod * tiles + pm * grid_n + pn numbers the
// (product, tile) pair. The XCD
// renumbering runs over all workgroups of the launch, so the ids one XCD
// serves are consecutive tiles of one product and K range.
struct WorkItem {
    int pm, pn, split, prod, slot;
};

__host__ __device__ inline WorkItem work_item(int wg, const GemmArgs &g) {
    const int tiles = g.grid_m * g.grid_n;
    const int total = tiles * g.splits * g.batch;  // < 2^31, checked on the host
    const int lid = (g.xcd_remap && g.num_xcd > 1) ? xcd_rank(wg, total, g.num_xcd) : wg;
    WorkItem w;
    const int t = lid % tiles;
    const int rest = lid / tiles;
    w.split = rest % g.splits;
    w.prod = rest / g.splits;
    group_major(t, g.grid_m, g.grid_n, g.group_m, w.pm, w.pn);
    w.slot = w.prod * tiles + w.pm * g.grid_n + w.pn;  // row-major tile number: independent of launch order
    return w;
}

// Bytes of the stream-K flags at the start of the workspace (one 8-byte flag
// per rank, padded to 256 bytes); the partial tiles follow.
__host__ __device__ inline int64_t sk_flag_bytes(int groups) { return ((int64_t)groups * 8 + 255) / 256 * 256; }

// Workgroups of one launch.
inline unsigned launch_groups(const GemmArgs &g) {
    if (g.sk_groups > 0) return (unsigned)g.sk_groups;
    return (unsigned)g.grid_m * (unsigned)g.grid_n * (unsigned)g.splits * (unsigned)g.batch;
}

}  // namespace dg
