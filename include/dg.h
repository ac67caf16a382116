/*
 * dg.h -- C-ABI of an MI355X (gfx950) tiled dense matrix multiply.
 *
 *   C[i][j] = round_out( sum_{k<K} A[i][k] * B[k][j] ),  0 <= i < M, 0 <= j < N
 *
 * The operation is the product of an M x K matrix and a K x N matrix
 * ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到 MatMul", §3.1: an output
 * element is a row of A times a column of B, summed over K). Each workgroup
 * owns one BLOCK_M x BLOCK_N tile of C and walks K in BLOCK_K slices
 * (same page §3.2-§3.4; "Triton：04 Matmul、Autotune 与 PyTorch 集成", the tile
 * view), accumulating in fp32 ("I Wrote a GPU Matmul Kernel From Scratch in
 * Triton", the finding that fp32 accumulation matters; load fp16, accumulate
 * fp32, store fp16 or fp32).
 *
 * Conventions for every entry point that takes a problem:
 *  - Pointers A, B, C are DEVICE pointers (HIP device memory), owned by the
 *    caller. The library never allocates device memory on the dg_gemm path
 *    and never frees caller memory.
 *  - Strides are in ELEMENTS, not bytes ("用 Triton 写 GPU Kernel" §4.1): A[i][k]
 *    is at A + i*stride_am + k*stride_ak, B[k][j] at B + k*stride_bk +
 *    j*stride_bn, C[i][j] at C + i*stride_cm + j*stride_cn. This is the
 *    stride-argument form of the teaching kernel in "Triton：04 Matmul…".
 *    A and B strides must be >= 0 (0 is allowed: a broadcast operand). C
 *    strides must be >= 1 and C's index map injective (no two (i, j) share
 *    an element).
 *  - Accumulation is fp32; inputs of fp16/bf16 give exact products. The
 *    output is rounded to out_dtype with round-to-nearest-even (the pages
 *    cast the fp32 accumulator to the output type after the K loop).
 *  - A and B are read only inside their M x K / K x N views; elements past a
 *    ragged edge count as zero (the masked load with other = 0 of the
 *    pages' kernels). Every element of C's M x N view is written exactly
 *    once; nothing else in C's allocation is written. dg_gemm and
 *    dg_gemm_config overwrite C; dg_gemm_ex adds alpha, beta, a residual, a
 *    bias and an activation.
 *  - M == 0 or N == 0: returns DG_OK and launches nothing. K == 0: C is
 *    filled with +0 (the empty sum).
 *  - stream is a hipStream_t (NULL = the legacy default stream). Work is
 *    enqueued on it; dg_gemm returns without synchronising the host.
 *  - On any error the call returns a status != DG_OK, enqueues nothing, and
 *    dg_last_error() describes it (thread-local).
 *  - All entry points are thread-safe; the config cache is mutex-guarded.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_dtype {
    DG_F32 = 0,   /* IEEE binary32 */
    DG_F16 = 1,   /* IEEE binary16 */
    DG_BF16 = 2   /* bfloat16 (top half of a binary32) */
} dg_dtype;

typedef enum dg_status {
    DG_OK = 0,
    DG_ERR_INVALID_VALUE = 1,  /* bad dimension, pointer, stride, alignment or dtype */
    DG_ERR_UNSUPPORTED = 2,    /* valid request the library has no kernel for */
    DG_ERR_NO_CONFIG = 3,      /* explicit config invalid for this problem/dtype */
    DG_ERR_HIP = 4             /* a HIP runtime call failed */
} dg_status;

/* Kernel families (dg_config.variant). */
enum {
    DG_VARIANT_SIMT = 0,  /* LDS-tiled fp32 FMA kernel: any dtype pair, any strides */
    DG_VARIANT_MFMA = 1   /* matrix cores, fp32 accumulators: v_mfma_f32_32x32x16 for fp16/bf16
                             inputs, v_mfma_f32_32x32x2_f32 for fp32 inputs */
};

/*
 * One kernel configuration. The tile sizes, waves and stages name a kernel
 * instantiation compiled into the library (block sizes are compile-time, as
 * in the pages' constexpr BLOCK_M/N/K); group_m and xcd_remap are read at
 * launch time.
 *  block_m, block_n, block_k: tile of C per workgroup and K slice per step.
 *  group_m:   rows of tiles per group in the group-major launch order
 *             ("I Wrote a GPU Matmul Kernel From Scratch in Triton", Step 4);
 *             1 gives plain row-major tile order.
 *  waves:     64-lane wavefronts per workgroup (the num_warps analogue).
 *  stages:    LDS buffers in the K pipeline (num_stages analogue; 2 = load
 *             slice s+1 while slice s is multiplied, S = keep S-1 slices in
 *             flight). Operands that need element-wise loads (unaligned or
 *             non-unit-stride layouts) always run a two-buffer pipeline;
 *             for them the value is not used.
 *  variant:   DG_VARIANT_*.
 *  xcd_remap: 1 = reorder workgroup ids so the tiles dispatched to one XCD
 *             (one L2) are consecutive in the group-major order.
 *  k_splits:  1 (or 0) = one workgroup walks all of K for its tile; S > 1 =
 *             split-K: S workgroups per tile each walk one K range of
 *             block_k-multiple length and store an fp32 partial tile; a
 *             second kernel sums the partials in range order (deterministic)
 *             and runs the epilogue. Needs a workspace (dg_gemm_ex); MFMA
 *             kernels only.
 *             DG_STREAM_K = stream-K: one workgroup per CU (at most two
 *             per tile). Each computes whole tiles while more than one
 *             whole round of one tile per CU remains; the K steps of the
 *             rest (the last, partial round and one whole round before it,
 *             or every tile when there are fewer tiles than CUs) are shared
 *             out evenly over the workgroups, so a tile is cut into at most
 *             three pieces; a tile's owner adds the other workgroups' fp32
 *             partials in K order (deterministic) and runs the epilogue.
 *             One kernel; needs a workspace (dg_gemm_ex). MFMA kernels with
 *             block_k 64 and block 64x64 (4 stages for the direct-to-LDS
 *             kernel, 2 otherwise) or 128x128 (2 stages).
 *             Splitting K follows from a tile being the sum of its K-slice
 *             partials ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到
 *             MatMul" §3.3); sharing out the partial last round answers the
 *             shape-dependence of the best config ("Triton：04 Matmul、
 *             Autotune 与 PyTorch 集成").
 */
#define DG_STREAM_K (-1)
typedef struct dg_config {
    int32_t block_m, block_n, block_k;
    int32_t group_m;
    int32_t waves;
    int32_t stages;
    int32_t variant;
    int32_t xcd_remap;
    int32_t k_splits;
} dg_config;

/*
 * C = A @ B with the library's choice of kernel: the cached config for this
 * problem key if one exists (see dg_autotune), else a built-in heuristic.
 * This is the pages' host wrapper, which checks the shapes, computes the
 * grid from the block sizes and launches the kernel ("用 Triton 写 GPU
 * Kernel：从 Vector Add、Softmax 到 MatMul" §4.5; the kernel's runtime arguments
 * are the pointers, M, N, K and the strides of "Triton：04 Matmul、Autotune 与
 * PyTorch 集成", its teaching kernel), with C supplied by the caller.
 * Never benchmarks, so its cost is one kernel launch (unless the
 * environment sets DG_AUTOTUNE_ON_MISS=1, which autotunes on a cache miss,
 * as the pages' first call does).
 * Arguments: problem sizes; the three device pointers and their element
 * strides; the input dtype (shared by A and B) and the output dtype; stream.
 * Errors: DG_ERR_INVALID_VALUE / DG_ERR_UNSUPPORTED from the checks listed
 * at the top of this file, DG_ERR_HIP if the launch fails; nothing is
 * enqueued on error.
 */
dg_status dg_gemm(int64_t M, int64_t N, int64_t K,
                  const void *A, int64_t stride_am, int64_t stride_ak,
                  const void *B, int64_t stride_bk, int64_t stride_bn,
                  void *C, int64_t stride_cm, int64_t stride_cn,
                  dg_dtype in_dtype, dg_dtype out_dtype, void *stream);

/*
 * Same as dg_gemm with an explicit configuration (tests, ablations): one
 * point of the autotune space, i.e. the block sizes, warps (here waves) and
 * pipeline stages that a configuration fixes ("Triton：04 Matmul、Autotune 与
 * PyTorch 集成", the section on what autotune chooses; "I Wrote a GPU Matmul
 * Kernel From Scratch in Triton", Step 3, which launches with one fixed block
 * size). A config that names no compiled kernel, or one that cannot run this
 * problem's dtype pair, returns DG_ERR_NO_CONFIG. The problem size is never
 * a reason to reject a config: ragged edges and K < block_k are masked
 * ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到 MatMul" §4.5-§4.6, the
 * masked loads and store).
 */
dg_status dg_gemm_config(int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t stride_am, int64_t stride_ak,
                         const void *B, int64_t stride_bk, int64_t stride_bn,
                         void *C, int64_t stride_cm, int64_t stride_cn,
                         dg_dtype in_dtype, dg_dtype out_dtype, void *stream,
                         const dg_config *cfg);

/*
 * Benchmark every candidate config for this problem on the caller's buffers
 * (C is overwritten many times), keep the fastest (lowest median of
 * `repeats` timed launches after warm-up; ties go to the earlier candidate),
 * store it in the cache under the problem key, and run it once more so C
 * holds its result. Synchronises `stream`. This is the pages' autotune:
 * measure candidate configs for a shape key and cache the winner
 * ("Triton：04 Matmul、Autotune 与 PyTorch 集成", what autotune chooses).
 * chosen / best_ms may be NULL. repeats <= 0 selects a default.
 */
dg_status dg_autotune(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t stride_am, int64_t stride_ak,
                      const void *B, int64_t stride_bk, int64_t stride_bn,
                      void *C, int64_t stride_cm, int64_t stride_cn,
                      dg_dtype in_dtype, dg_dtype out_dtype, void *stream,
                      int32_t repeats, dg_config *chosen, float *best_ms);

/* Activation applied last by a fused epilogue. */
typedef enum dg_activation {
    DG_ACT_NONE = 0,
    DG_ACT_RELU = 1,  /* v < 0 ? +0 : v (NaN and -0 pass through) */
    DG_ACT_GELU = 2   /* v * Phi(v), Phi the standard normal CDF (the erf form) */
} dg_activation;

/*
 * Fused epilogue:
 *
 *   C[i][j] = act(alpha * (A @ B)[i][j] + beta * R[i][j] + bias)
 *
 * evaluated in fp32 on the fp32 accumulator, then rounded once to C's dtype
 * (RNE). This is the element-wise work that follows the product when it
 * stands in for a linear layer ("如何用Triton手写Kernel优化矩阵乘与Flash
 * Attention？", 性能对比与工程落地建议), fused into the kernel that produces it
 * so the intermediate never goes to memory ("用 Triton 写 GPU Kernel：从 Vector
 * Add、Softmax 到 MatMul", §2.7).
 *  alpha:          scales the product.
 *  beta:           scales the residual R. beta == 0: R is not read at all
 *                  (so C's prior contents may be uninitialised, even NaN).
 *  residual:       NULL: R is C's prior contents (C's dtype and strides,
 *                  an in-place C = alpha*AB + beta*C). Else a DEVICE matrix
 *                  of residual_dtype with element strides (stride_rm,
 *                  stride_rn) >= 0 that must not overlap C's view.
 *  bias:           NULL, or a DEVICE vector of bias_dtype with element
 *                  stride bias_stride (>= 0): bias[j] for column j (length N)
 *                  if bias_per_row == 0, else bias[i] for row i (length M).
 *  activation:     dg_activation.
 * A NULL dg_epilogue means alpha = 1, beta = 0, no bias, no activation.
 */
typedef struct dg_epilogue {
    float alpha;
    float beta;
    const void *residual;
    int32_t residual_dtype;
    int64_t stride_rm, stride_rn;
    const void *bias;
    int32_t bias_dtype;
    int32_t bias_per_row;
    int64_t bias_stride;
    int32_t activation;
} dg_epilogue;

/*
 * Strided batch of `count` independent products of the same shape:
 * product b reads A + b*stride_a, B + b*stride_b, residual + b*stride_r,
 * bias + b*stride_bias and writes C + b*stride_c (element strides, >= 0; 0
 * shares an operand across the batch). The C matrices of different products
 * must not overlap: with count > 1, C's (batch, row, column) strides sorted
 * by size must nest (each at least the span of the smaller ones), or
 * stride_c must be at least the span of one C view. count == 0 is a no-op.
 * A NULL dg_batch means count = 1. The transposed products of a backward
 * pass (dA = dC B^T, dB = A^T dC) are plain calls with swapped strides.
 */
typedef struct dg_batch {
    int64_t count;
    int64_t stride_a, stride_b, stride_c;
    int64_t stride_r, stride_bias;
} dg_batch;

/*
 * The general entry point: dg_gemm / dg_gemm_config plus an optional fused
 * epilogue, an optional strided batch, an optional explicit config (NULL:
 * the library's choice, as dg_gemm) and an optional workspace.
 *
 * workspace / workspace_bytes: DEVICE memory, 256-byte aligned, for split-K
 * (config k_splits > 1) and stream-K (k_splits = DG_STREAM_K); size from
 * dg_workspace_size. NULL / 0 if none.
 * With cfg == NULL and a workspace, the library may choose split-K for
 * problems whose output tiles leave most of the GPU idle and whose K is long,
 * when the workspace is large enough; without one it never splits. It never
 * chooses stream-K by itself (measured slower than the unsplit kernels on
 * MI355X); dg_autotune_ex times it. Split-K runs as two kernels on
 * `stream`: the K ranges store fp32 partial tiles in the workspace, then a
 * reduction kernel adds each tile's partials in range order (deterministic)
 * and applies the epilogue. Stream-K is one kernel; it keeps its partial
 * tiles and per-workgroup flags in the workspace (each launch writes its own
 * flag values, so nothing needs resetting). The workspace needs no
 * initialisation. Calls that share a workspace must not run concurrently
 * (issue them on one stream, or synchronise). The library never allocates.
 * An explicit config with k_splits > 1 or DG_STREAM_K and no (or too small a)
 * workspace is DG_ERR_INVALID_VALUE; with a SIMT config, or DG_STREAM_K on a
 * tile shape compiled without it, it is DG_ERR_NO_CONFIG.
 */
dg_status dg_gemm_ex(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t stride_am, int64_t stride_ak,
                     const void *B, int64_t stride_bk, int64_t stride_bn,
                     void *C, int64_t stride_cm, int64_t stride_cn,
                     dg_dtype in_dtype, dg_dtype out_dtype, void *stream,
                     const dg_epilogue *epilogue, const dg_batch *batch,
                     const dg_config *cfg, void *workspace, int64_t workspace_bytes);

/*
 * dg_gemm_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments and results as dg_gemm_ex, without the workspace: split-K
 * partial tiles go to a scratch array inside the library, a file-scope
 * device array of DG_NOALLOC_SCRATCH_BYTES per GPU that exists from the
 * library's load until the process ends. Nothing is allocated or freed.
 *  - cfg == NULL: the library's choice, as dg_gemm_ex with a workspace of
 *    DG_NOALLOC_SCRATCH_BYTES (it splits K only when the partials fit).
 *  - An explicit cfg whose partials need more than DG_NOALLOC_SCRATCH_BYTES
 *    (dg_workspace_size) returns DG_ERR_UNSUPPORTED and enqueues nothing.
 *  - Every call on one GPU shares that GPU's scratch. Calls whose split-K
 *    work overlaps in time on one GPU (different streams or threads without
 *    synchronisation) race and give wrong results: issue them on one stream
 *    or synchronise. The partials need no initialisation (each is written
 *    before it is read, within the call).
 *  - The first call on a device looks up that device's copy of the array
 *    (hipGetSymbolAddress with the device current); DG_ERR_HIP if it fails.
 */
#define DG_NOALLOC_SCRATCH_BYTES (32 << 20)
dg_status dg_gemm_ex_noalloc(int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t stride_am, int64_t stride_ak,
                             const void *B, int64_t stride_bk, int64_t stride_bn,
                             void *C, int64_t stride_cm, int64_t stride_cn,
                             dg_dtype in_dtype, dg_dtype out_dtype, void *stream,
                             const dg_epilogue *epilogue, const dg_batch *batch,
                             const dg_config *cfg);

/*
 * dg_autotune for a dg_gemm_ex problem (epilogue and batch included in every
 * timed launch). With a workspace, the candidates also include split-K
 * counts (2, 4, 8, 16) for tile shapes that do not fill the GPU, and
 * stream-K for tile shapes whose last round of tiles is partial. The winner
 * is cached under (M, N, K, batch count, dtypes, layouts); a later dg_gemm_ex
 * with cfg == NULL uses it (unsplit if that call's workspace is too small).
 * An epilogue that reads C (beta != 0 and no separate residual) is
 * rejected with DG_ERR_INVALID_VALUE: every trial launch would change C.
 */
dg_status dg_autotune_ex(int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t stride_am, int64_t stride_ak,
                         const void *B, int64_t stride_bk, int64_t stride_bn,
                         void *C, int64_t stride_cm, int64_t stride_cn,
                         dg_dtype in_dtype, dg_dtype out_dtype, void *stream,
                         const dg_epilogue *epilogue, const dg_batch *batch,
                         void *workspace, int64_t workspace_bytes,
                         int32_t repeats, dg_config *chosen, float *best_ms);

/*
 * Workspace bytes config `cfg` needs for an M x N x K problem with
 * `batch_count` products. Split-K rests on the K slices of one output tile
 * adding up to its value in any grouping ("用 Triton 写 GPU Kernel：从 Vector
 * Add、Softmax 到 MatMul" §3.3, where tile (0, 0) is the sum of two K-slice
 * partials); each range's partial tile is kept here until it is summed.
 * Sizes: 0 when it does not split K, else one fp32 partial
 * tile per (product, tile, K range) = tiles * batch_count * ranges *
 * block_m * block_n * 4. K is cut into ranges of k_chunk = block_k *
 * ceil(ceil(K / k_splits) / block_k) elements; the ranges actually used
 * number ceil(K / k_chunk) (at most k_splits; 1 when K <= block_k).
 * Stream-K (k_splits = DG_STREAM_K): with G = the current device's CU count,
 * 8 * G bytes of flags rounded up to 256, then G partial tiles of
 * block_m * block_n * 4 bytes (0 for an empty problem).
 */
dg_status dg_workspace_size(int64_t M, int64_t N, int64_t K, int64_t batch_count, const dg_config *cfg,
                            int64_t *bytes);

/*
 * Attention forward: for every batch b and head h,
 *
 *   O[i][:] = sum_j softmax_j(scale * Q[i]·K[j]) V[j][:],   lse[i] = log sum_j exp(scale * Q[i]·K[j])
 *
 * over the allowed keys j (all j < seq_kv; with causal != 0 only j <= i).
 * This is the blockwise, online-softmax attention of "如何用Triton手写Kernel优化
 * 矩阵乘与Flash Attention？" (its Flash Attention section): one program per
 * query block walks the key blocks keeping a running maximum and sum, so
 * the score matrix is never stored.
 *  Q: [batch][heads][seq_q][head_dim]; K, V: [batch][heads][seq_kv][head_dim];
 *     O: [batch][heads][seq_q][head_dim]. DEVICE pointers; each *_strides is
 *     a host array of 3 element strides (batch, head, seq); the head_dim
 *     stride is 1. Q, K, V (in_dtype, fp16 or bf16) need 16-byte aligned
 *     bases and batch/head/seq strides that are multiples of 8 elements.
 *  lse: NULL, or a DEVICE fp32 array [batch][heads][seq_q] (contiguous) that
 *     receives the natural-log sum of exponentials per query (-inf for a query
 *     with no allowed key).
 *  out_dtype: O's dtype (f32, f16 or bf16), rounded from the fp32 result.
 *  scale: the score scale; <= 0 (or NaN) selects 1 / sqrt(head_dim).
 *  Numerics: fp32 scores, softmax and accumulation; the softmax weights are
 *     rounded to in_dtype for the product with V (the matrix cores take 16-bit
 *     operands); the normalising sum uses the unrounded weights.
 *  Supported: head_dim 64 and 128. Other head_dim values, in_dtype f32, or layouts
 *     outside the above return DG_ERR_UNSUPPORTED; bad arguments return
 *     DG_ERR_INVALID_VALUE. Any size may be 0 (nothing to do; seq_kv == 0
 *     writes O = 0 and lse = -inf). seq_q, seq_kv < 2^30.
 */
dg_status dg_attention_fwd(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_kv, int64_t head_dim,
                           const void *Q, const int64_t *q_strides, const void *K, const int64_t *k_strides,
                           const void *V, const int64_t *v_strides, void *O, const int64_t *o_strides,
                           float *lse, dg_dtype in_dtype, dg_dtype out_dtype, float scale, int32_t causal,
                           void *stream);

/*
 * The config dg_gemm would use, without any GPU work. The pointers are only
 * inspected for alignment (they may be NULL: then taken as 16-byte aligned).
 * *from_cache (may be NULL) is set to 1 if the config came from the cache.
 * The cache key is (M, N, K) plus the dtypes, each operand's layout class
 * and the vector-alignment class: the pages key the tuned choice on M, N and
 * K and tune again when any of them changes ("I Wrote a GPU Matmul Kernel
 * From Scratch in Triton", Step 5), and keep the winner per input size
 * ("Triton：04 Matmul、Autotune 与 PyTorch 集成", the section on what autotune
 * chooses). A miss falls back to a heuristic, since different shapes want
 * different configs (same page, the section on why shapes need different
 * configs).
 */
dg_status dg_select_config(int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t stride_am, int64_t stride_ak,
                           const void *B, int64_t stride_bk, int64_t stride_bn,
                           const void *C, int64_t stride_cm, int64_t stride_cn,
                           dg_dtype in_dtype, dg_dtype out_dtype,
                           dg_config *out, int32_t *from_cache);

/*
 * The config dg_gemm_ex would use with cfg == NULL for this batch (NULL: one
 * product) and a workspace of workspace_bytes (split-K is chosen only when
 * its workspace fits), without any GPU work. Pointers, key and citations as
 * dg_select_config; the batch count is part of the key.
 */
dg_status dg_select_config_ex(int64_t M, int64_t N, int64_t K,
                              const void *A, int64_t stride_am, int64_t stride_ak,
                              const void *B, int64_t stride_bk, int64_t stride_bn,
                              const void *C, int64_t stride_cm, int64_t stride_cn,
                              dg_dtype in_dtype, dg_dtype out_dtype, const dg_batch *batch,
                              int64_t workspace_bytes, dg_config *out, int32_t *from_cache);

/*
 * Autotune candidates for a dtype pair: count, and the i-th (0-based). The
 * pages tune over an explicit list of configs ("I Wrote a GPU Matmul Kernel
 * From Scratch in Triton", Step 5, fifteen of them) and note that autotune
 * can only pick among the candidates it is given ("Triton：04 Matmul、Autotune
 * 与 PyTorch 集成", the second common mistake). dg_get_candidate returns
 * DG_ERR_INVALID_VALUE for an index outside [0, count) or an unknown dtype;
 * dg_num_candidates returns 0 for an unknown dtype.
 */
int32_t dg_num_candidates(dg_dtype in_dtype, dg_dtype out_dtype);
dg_status dg_get_candidate(int32_t i, dg_dtype in_dtype, dg_dtype out_dtype, dg_config *out);

/*
 * Check a full argument list exactly as dg_gemm does, without launching. The
 * pages' wrapper asserts that the inner dimensions agree and the inputs are
 * contiguous before it launches ("用 Triton 写 GPU Kernel：从 Vector Add、
 * Softmax 到 MatMul" §4.5); here a failed check is a status code (DG_OK or
 * DG_ERR_INVALID_VALUE / DG_ERR_UNSUPPORTED) plus dg_last_error(), and any
 * strides are accepted as long as C's index map is injective.
 */
dg_status dg_validate(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t stride_am, int64_t stride_ak,
                      const void *B, int64_t stride_bk, int64_t stride_bn,
                      const void *C, int64_t stride_cm, int64_t stride_cn,
                      dg_dtype in_dtype, dg_dtype out_dtype);

/*
 * Launch-order helper (host side of the device tile map): the C tile
 * (*pid_m, *pid_n) that workgroup `wg` computes, for a grid of
 * grid_m x grid_n tiles, group_m rows per group (group-major order, "I Wrote
 * a GPU Matmul Kernel From Scratch in Triton", Step 4) and, if xcd_remap, the
 * XCD-aware renumbering over num_xcd XCDs. Returns DG_ERR_INVALID_VALUE for
 * wg outside [0, grid_m*grid_n) or non-positive sizes.
 */
dg_status dg_tile_coords(int32_t grid_m, int32_t grid_n, int32_t group_m, int32_t xcd_remap,
                         int32_t num_xcd, int32_t wg, int32_t *pid_m, int32_t *pid_n);

/*
 * Grid a config launches for a problem: tiles along M and N, and K steps
 * (ceil divisions, "用 Triton 写 GPU Kernel" §3.2 and §4.6).
 */
dg_status dg_grid_shape(int64_t M, int64_t N, int64_t K, const dg_config *cfg,
                        int64_t *grid_m, int64_t *grid_n, int64_t *k_steps);

/*
 * Config cache: the winners of dg_autotune / dg_autotune_ex under their keys
 * (the pages cache the fastest config per key, so that only the first call
 * at a shape pays for the benchmark: "I Wrote a GPU Matmul Kernel From
 * Scratch in Triton", Step 5; "Triton：04 Matmul、Autotune 与 PyTorch 集成", the
 * section on what autotune chooses). dg_cache_clear empties it;
 * dg_cache_save writes it to a text file (a header line, then one key and
 * config per line) and dg_cache_load merges such a file into it, skipping
 * malformed lines (their count goes to dg_last_error). Save/load return
 * DG_ERR_INVALID_VALUE for a NULL path, a file that cannot be opened or
 * written, or a file without the header. dg_cache_size counts the entries.
 * Mutex-guarded; the cache lives in host memory for the process.
 */
dg_status dg_cache_clear(void);
dg_status dg_cache_save(const char *path);
dg_status dg_cache_load(const char *path);
int32_t dg_cache_size(void);

/*
 * Static description of a status code, and the calling thread's last error
 * (an empty string after a successful call). The pages stop a bad call with
 * an assert ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到 MatMul" §4.5);
 * a C library returns the status instead and keeps the detail here. Both
 * strings are owned by the library: the first is static, the second valid
 * until the thread's next call into the library.
 */
const char *dg_status_string(dg_status s);
const char *dg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
