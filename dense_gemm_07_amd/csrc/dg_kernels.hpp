// Device code of the dense GEMM library (gfx950 / CDNA4).
//
// Two kernel families, both "one workgroup per BLOCK_M x BLOCK_N tile of C,
// walk K in BLOCK_K slices, accumulate in fp32, mask ragged edges"
// ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到 MatMul" §3.2-§3.4 and
// §4.5-§4.6; "Triton：04 Matmul、Autotune 与 PyTorch 集成", the tile view):
//
//  gemm_simt  -- scalar fp32 FMA over LDS tiles. Any dtype pair, any strides
//                and alignment. Used for fp32 inputs and as the fallback.
//  gemm_mfma  -- fp16/bf16 inputs on v_mfma_f32_32x32x16 matrix cores with
//                fp32 accumulators, a two-buffer LDS pipeline (slice s+1 is
//                fetched while slice s is multiplied), padded LDS rows, and a
//                masked, dtype-converting epilogue.
//  gemm_mfma_lds -- the same tiles with operands moved global -> LDS by the
//                buffer unit and an S-stage pipeline.
//
// Every kernel also serves a strided batch of products, an optional fused
// epilogue (C = act(alpha * acc + beta * R + bias)), and -- the MFMA kernels
// -- split-K with a deterministic reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_internal.hpp"

namespace dg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- element conversions -----------------------------------------------------

// Storage tags: the element type of A/B/C in memory.
struct F32 { using storage = float; static constexpr int code = DG_F32; };
struct F16 { using storage = uint16_t; static constexpr int code = DG_F16; };
struct BF16 { using storage = uint16_t; static constexpr int code = DG_BF16; };

template <typename T> __device__ __forceinline__ float to_f32(typename T::storage v);
template <> __device__ __forceinline__ float to_f32<F32>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<F16>(uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
}
template <> __device__ __forceinline__ float to_f32<BF16>(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);  // bf16 is the top half of an fp32
}

// fp32 -> storage, round to nearest even (the hardware conversions).
template <typename T> __device__ __forceinline__ typename T::storage from_f32(float v);
template <> __device__ __forceinline__ float from_f32<F32>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<F16>(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <> __device__ __forceinline__ uint16_t from_f32<BF16>(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---- fused epilogue ----------------------------------------------------------
// The element-wise work after the K loop runs on the fp32 accumulator before
// the single rounding to C's dtype, so an activation or bias costs no extra
// pass over C ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到 MatMul" §2.7:
// fusion keeps intermediates on chip and saves launches).

__device__ __forceinline__ float load_any(const void *p, int64_t off, int dt) {
    if (dt == DG_BF16) return to_f32<BF16>(static_cast<const uint16_t *>(p)[off]);
    if (dt == DG_F16) return to_f32<F16>(static_cast<const uint16_t *>(p)[off]);
    return static_cast<const float *>(p)[off];
}

// Upper tail of the standard normal, Q(x) = Phi(-x), for x >= 0:
// exp(-x^2/2) * t * P(t) with t = 1 / (1 + 0.3 x) and P of degree 9, fitted
// to 3.5e-9 relative error on [0, 14] (fit_normal_tail.py). x^2 is carried
// as hi + lo so the exponent is exact to fp32 rounding; no branches, so a
// wave whose lanes fall in different ranges runs it once. Measured end to
// end in fp32 emulation: <= 7 ulp relative where the result is normal.
__device__ __forceinline__ float normal_tail(float x) {
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3f * x);  // hardware reciprocal, 1 ulp
    float p = -0.0206153598f;
    p = __builtin_fmaf(p, t, 0.11239133f);
    p = __builtin_fmaf(p, t, -0.228108361f);
    p = __builtin_fmaf(p, t, 0.191641822f);
    p = __builtin_fmaf(p, t, -0.0793019533f);
    p = __builtin_fmaf(p, t, 0.0960895121f);
    p = __builtin_fmaf(p, t, 0.0784138665f);
    p = __builtin_fmaf(p, t, 0.110229976f);
    p = __builtin_fmaf(p, t, 0.119572505f);
    p = __builtin_fmaf(p, t, 0.119686648f);
    // exp(-x^2/2) = 2^(-x^2 log2(e) / 2) with the exponent carried as
    // a_hi + a_lo (x^2 = hi + lo exactly, and the product by log2(e)/2 keeps
    // its rounding error), so v_exp_f32 sees an argument exact to fp32.
    const float hi = x * x;
    const float lo = __builtin_fmaf(x, x, -hi);
    constexpr float kL = -0.72134752044448170368f;  // -log2(e) / 2
    const float a_hi = hi * kL;
    const float a_lo = __builtin_fmaf(hi, kL, -a_hi) + lo * kL;
    const float e = __builtin_amdgcn_exp2f(a_hi) * __builtin_fmaf(a_lo, 0.69314718055994530942f, 1.0f);
    return e * t * p;
}

// The same tail for results that are rounded to a 16-bit type: P of degree
// 6 (3.8e-6 relative error on [0, 14], fit_normal_tail.py --degree 6) and a
// plain fp32 exponent (relative error about 5e-8 * x^2). Below 1.5e-5
// relative wherever Q is an fp32 normal, which is under 1/16 of half an ulp
// of fp16 and 1/130 of bf16's: at most a rare last-bit difference after
// rounding, for a third fewer operations.
__device__ __forceinline__ float normal_tail_16(float x) {
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3f * x);
    float p = -0.0124396523f;
    p = __builtin_fmaf(p, t, -0.0353136659f);
    p = __builtin_fmaf(p, t, 0.160478696f);
    p = __builtin_fmaf(p, t, 0.0202635769f);
    p = __builtin_fmaf(p, t, 0.131027669f);
    p = __builtin_fmaf(p, t, 0.116067156f);
    p = __builtin_fmaf(p, t, 0.119914405f);
    return __builtin_amdgcn_exp2f(x * x * -0.72134752044448170368f) * t * p;
}

// ReLU keeps NaN and -0 (only v < 0 becomes +0). GELU is v * Phi(v), with
// Phi(v) = 1 - Q(v) for v >= 0 and Q(-v) below: no cancellation for large
// negative v. |v| is clamped at 30, where Q is exactly 0 in fp32, so
// GELU(+inf) = +inf and GELU(-inf) = -inf * 0 = NaN (the limit form's value).
__device__ __forceinline__ float activate(float v, int act) {
    if (act == DG_ACT_RELU) return v < 0.0f ? 0.0f : v;
    if (act == DG_ACT_GELU) {
        const float q = normal_tail(fminf(fabsf(v), 30.0f));
        return v * (v >= 0.0f ? 1.0f - q : q);
    }
    return v;
}

// GELU for a result that is rounded to bf16 or fp16 next (the fused
// epilogue's 16-bit outputs); an internal activation code, not in the ABI.
constexpr int kActGelu16 = 100;
__device__ __forceinline__ float gelu_16(float v) {
    const float q = normal_tail_16(fminf(fabsf(v), 30.0f));
    return v * (v >= 0.0f ? 1.0f - q : q);
}

// C[gm, gn] = act(alpha * v + beta * R[gm, gn] + bias) for one element.
// r_off / b_off are the batch offsets of R and bias.
__device__ __forceinline__ float epilogue_value(const GemmArgs &g, float v, int gm, int gn, int64_t r_off,
                                                int64_t b_off) {
    float x = g.alpha * v;
    if (g.beta != 0.0f) x = __builtin_fmaf(g.beta, load_any(g.R, r_off + (int64_t)gm * g.srm + (int64_t)gn * g.srn, g.r_dtype), x);
    if (g.bias) x += load_any(g.bias, b_off + (int64_t)(g.bias_per_row ? gm : gn) * g.sbias, g.bias_dtype);
    return activate(x, g.act);
}

// ============================================================================
// gemm_simt: 256 threads, a 16 x 16 thread grid, each thread RM x RN outputs.
// ============================================================================
template <typename TI, typename TO, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void gemm_simt(GemmArgs g) {
    constexpr int T = 256;
    constexpr int RM = BM / 16, RN = BN / 16;
    static_assert(BM % 16 == 0 && BN % 16 == 0, "tile must be a multiple of the 16x16 thread grid");
    __shared__ float As[BK][BM + 1];
    __shared__ float Bs[BK][BN + 1];

    const WorkItem w = work_item(blockIdx.x, g);  // the host launches this kernel with splits == 1
    const int m0 = w.pm * BM, n0 = w.pn * BN;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    using SI = typename TI::storage;
    using SO = typename TO::storage;
    const SI *A = static_cast<const SI *>(g.A) + (int64_t)w.prod * g.bsa;
    const SI *B = static_cast<const SI *>(g.B) + (int64_t)w.prod * g.bsb;
    SO *C = static_cast<SO *>(g.C) + (int64_t)w.prod * g.bsc;

    float acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < g.K; k0 += BK) {
        // Stage A[m0:m0+BM, k0:k0+BK] and B[k0:k0+BK, n0:n0+BN]; out-of-view
        // elements are zero and are not read.
        for (int e = tid; e < BM * BK; e += T) {
            const int r = e / BK, kk = e % BK;
            const int gm = m0 + r, gk = k0 + kk;
            float v = 0.0f;
            if (gm < g.M && gk < g.K) v = to_f32<TI>(A[(int64_t)gm * g.sam + (int64_t)gk * g.sak]);
            As[kk][r] = v;
        }
        for (int e = tid; e < BK * BN; e += T) {
            const int kk = e / BN, c = e % BN;
            const int gk = k0 + kk, gn = n0 + c;
            float v = 0.0f;
            if (gk < g.K && gn < g.N) v = to_f32<TI>(B[(int64_t)gk * g.sbk + (int64_t)gn * g.sbn]);
            Bs[kk][c] = v;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < BK; ++kk) {
            float a[RM], b[RN];
#pragma unroll
            for (int i = 0; i < RM; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < RN; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }

    const int64_t r_off = (int64_t)w.prod * g.bsr, b_off = (int64_t)w.prod * g.bsbias;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
        const int gm = m0 + ty + 16 * i;
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            const int gn = n0 + tx + 16 * j;
            if (gm < g.M && gn < g.N) {
                const float v = g.epi ? epilogue_value(g, acc[i][j], gm, gn, r_off, b_off) : acc[i][j];
                C[(int64_t)gm * g.scm + (int64_t)gn * g.scn] = from_f32<TO>(v);
            }
        }
    }
}

// ============================================================================
// gemm_mfma
// ============================================================================

// v_mfma_f32_32x32x16_{bf16,f16}: D[32x32] += A[32x16] * B[16x32].
// Operand registers (8 x 16-bit per lane): lane l holds A[l % 32][8*(l/32) + e]
// and B[8*(l/32) + e][l % 32], e = 0..7. The k assignment only has to agree
// between A and B. Result: lane l, register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].
template <typename TI> struct Mfma;
template <> struct Mfma<BF16> {
    static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<F16> {
    static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

// Pack/unpack 8 x 16-bit values <-> one 16-byte register.
__device__ __forceinline__ u32x4 pack8(const uint16_t (&v)[8]) {
    u32x4 r;
    r.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    r.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    r.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    r.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    return r;
}

// 16 bytes from an address that is only element (2-byte) aligned. gfx950
// serves unaligned global vector loads; the compiler emits one
// global_load_dwordx4 for this.
typedef unsigned int u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
__device__ __forceinline__ u32x4 load16_unaligned(const uint16_t *p) {
    const u32x4_a2 v = *reinterpret_cast<const u32x4_a2 *>(p);
    return u32x4{v.x, v.y, v.z, v.w};
}

// Drops the first `sh` 16-bit elements of an 8-element chunk (element 0 is
// the lowest 16 bits) and fills the top with zeros; sh >= 8 gives zero.
__device__ __forceinline__ u32x4 drop_elems(u32x4 v, int sh) {
    const uint64_t lo = ((uint64_t)v.y << 32) | v.x, hi = ((uint64_t)v.w << 32) | v.z;
    const int s = 16 * min(sh, 8);  // 0..128 bits
    const uint64_t lo_a = s == 0 ? lo : ((lo >> (s & 63)) | (hi << ((64 - s) & 63)));  // s < 64
    const uint64_t lo_b = hi >> ((s - 64) & 63);                                        // 64 <= s < 128
    const uint64_t nlo = s < 64 ? lo_a : (s < 128 ? lo_b : 0);
    const uint64_t nhi = s < 64 ? (hi >> (s & 63)) : 0;
    return u32x4{(uint32_t)nlo, (uint32_t)(nlo >> 32), (uint32_t)nhi, (uint32_t)(nhi >> 32)};
}

// Fetches one operand tile (ROWS x BK, rows = M for A or N for B) from
// global memory into registers, then writes it to LDS as [ROWS][LDK] with k
// contiguous. Elements outside the operand's view (row >= rows_valid or
// k >= K) become +0 and are never read.
//  LD_KU: k stride 1. Whole 8-element chunks are one 16-byte load at any
//         element alignment; a chunk cut by K is loaded element by element.
//  LD_GN: anything else, element loads through both strides.
// Element offset of (row, k), k a multiple of 8, in the register kernel's LDS
// tile. BK 64: rows of LDK = BK + 8 elements (the 16-byte pad breaks the bank
// pattern of 128-byte rows). BK 32: unpadded 64-byte rows whose four 16-byte
// chunks are permuted by bits 2-3 of the row, so both the 16-byte writes (a
// 16-lane group covers 4 rows x 4 chunks) and the fragment reads (16 rows,
// one chunk) touch 64 distinct banks; the padded 80-byte rows put the writes
// of rows 0 and 3 on the same banks (measured on MI355X: 614 k conflict
// cycles of 1.84 M LDS cycles on the 1000x1500x777 product).
template <int BK, int LDK>
__device__ __forceinline__ int reg_lds_off(int row, int k) {
    if constexpr (BK == 32) return row * 32 + ((((k >> 3) ^ (row >> 2)) & 3) << 3);
    else return row * LDK + k;
}

template <int ROWS, int BK, int LDK, int T, int MODE>
struct TileLoader {
    // Row-contiguous unaligned operands (LD_RU) take the staged kernel at
    // every tile size.
    static_assert(MODE == LD_KU || MODE == LD_GN, "register-staged load modes");
    static constexpr int KCH = BK / 8;                   // 8-element k-chunks per row
    static constexpr int NCH = ROWS * KCH;               // chunks per tile
    static constexpr int PER = (NCH + T - 1) / T;

    u32x4 reg[PER];
    bool okc[PER];         // LD_KU: chunk c is inside the operand (else LDS gets zeros)
    const uint16_t *base;  // element (row0, k = 0) of the operand
    int64_t srow, sk;      // element strides along rows and along k
    int rows_valid;        // rows of the tile inside the operand
    int K;

    // INSIDE_K: the caller knows k0 + BK <= K. Then the loads have no branch:
    // a branch around a load (the element loads at the edges) makes the
    // compiler wait for the load where the two paths join, i.e. at once.
    // LD_KU chunks are one 16-byte load each from a row clamped into the
    // operand; the row mask is applied when the chunk is written to LDS
    // (store).
    template <bool INSIDE_K = false>
    __device__ __forceinline__ void load(int tid, int k0) {
        if constexpr (MODE == LD_KU && INSIDE_K) {
#pragma unroll
            for (int c = 0; c < PER; ++c) {
                const int q = c * T + tid;
                const int r = q / KCH, kc = q % KCH;
                okc[c] = ((NCH % T == 0) || q < NCH) && r < rows_valid;
                const int rr = r < rows_valid ? r : (rows_valid > 0 ? rows_valid - 1 : 0);
                reg[c] = load16_unaligned(base + (int64_t)rr * srow + k0 + kc * 8);
            }
            return;
        }
        if constexpr (MODE == LD_KU) {
#pragma unroll
            for (int c = 0; c < PER; ++c) okc[c] = true;
        }
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int q = c * T + tid;
            const int r = q / KCH, kc = q % KCH;
            const int k = k0 + kc * 8;
            const bool ok = ((NCH % T == 0) || q < NCH) && r < rows_valid;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (MODE == LD_KU) {
                const uint16_t *p = base + (int64_t)r * srow + k;
                if (ok && k + 8 <= K) {
                    v = load16_unaligned(p);
                } else if (ok && k < K) {
                    uint16_t e8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) e8[e] = (k + e < K) ? p[e] : (uint16_t)0;
                    v = pack8(e8);
                }
            } else {  // LD_GN
                if (ok) {
                    const uint16_t *p = base + (int64_t)r * srow;
                    uint16_t e8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) e8[e] = (k + e < K) ? p[(int64_t)(k + e) * sk] : (uint16_t)0;
                    v = pack8(e8);
                }
            }
            reg[c] = v;
        }
    }

    __device__ __forceinline__ void store(int tid, uint16_t *lds) const {
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int q = c * T + tid;
            if ((NCH % T == 0) || q < NCH) {
                const int r = q / KCH, kc = q % KCH;
                u32x4 v = reg[c];
                if constexpr (MODE == LD_KU) v = okc[c] ? v : u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4 *>(lds + reg_lds_off<BK, LDK>(r, kc * 8)) = v;
            }
        }
    }
};


// The loads of a k-contiguous operand tile (any element alignment) for the
// deep pipeline of the small register-staged tiles: P register sets, every
// chunk one 16-byte load with no branch, for any slice (also past K). The
// thread's chunk rows are clamped to the tile's last valid row and k to
// K - 8 (the caller guarantees that the operand has at least 8 columns, so
// k = K - 8 relative to a K range still lies inside the row); store() undoes
// both clamps: a chunk cut by K drops the elements it read before its own
// k, chunks past K and rows past the valid ones become zeros.
template <int ROWS, int BK, int LDK, int T, int P>
struct KuStream {
    static constexpr int KCH = BK / 8;      // 8-element k-chunks per row
    static constexpr int NCH = ROWS * KCH;  // chunks per tile
    static constexpr int PER = (NCH + T - 1) / T;
    u32x4 reg[P][PER];
    const uint16_t *row[PER];  // element (clamped row, k = chunk's k) of the operand
    int kmax;                  // K - 8
    int rows_valid;

    __device__ __forceinline__ void init(const uint16_t *base, int64_t srow, int rows, int K, int tid) {
        kmax = K - 8;
        rows_valid = rows;
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int q = c * T + tid;
            const int r = q / KCH;
            const int rr = r < rows ? r : rows - 1;
            row[c] = base + (int64_t)rr * srow;
        }
    }
    __device__ __forceinline__ void load(int set, int tid, int k0) {
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int k = k0 + ((c * T + tid) % KCH) * 8;
            reg[set][c] = load16_unaligned(row[c] + min(k, kmax));
        }
    }
    // TAIL: the slice reaches past K (only then can a chunk need its clamp undone).
    template <bool TAIL>
    __device__ __forceinline__ void store_t(int set, int tid, uint16_t *lds, int k0) const {
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int q = c * T + tid;
            if ((NCH % T == 0) || q < NCH) {
                const int r = q / KCH, kc = q % KCH;
                u32x4 v = reg[set][c];
                if constexpr (TAIL) {
                    const int k = k0 + kc * 8;
                    v = drop_elems(v, k - min(k, kmax));
                }
                if (r >= rows_valid) v = u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4 *>(lds + reg_lds_off<BK, LDK>(r, kc * 8)) = v;
            }
        }
    }
    __device__ __forceinline__ void store(int set, int tid, uint16_t *lds, int k0) const {
        if (k0 + BK > kmax + 8) store_t<true>(set, tid, lds, k0);
        else store_t<false>(set, tid, lds, k0);
    }
};

// Writes the accumulator tile (lane l, register r of block (i, j) is element
// (row_base + 32i + 8(r/4) + r%4, col_base + 32j)) to C, masked to C's view
// unless the tile is interior. c_off is the batch offset of C.
template <typename TO, int FM, int FN>
__device__ __forceinline__ void store_acc(const GemmArgs &g, int64_t c_off, const f32x16 (&acc)[FM][FN],
                                          int row_base, int col_base, bool interior) {
    typename TO::storage *C = static_cast<typename TO::storage *>(g.C) + c_off;
    if (interior) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t cbase = (int64_t)(col_base + j * 32) * g.scn;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gm = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    C[(int64_t)gm * g.scm + cbase] = from_f32<TO>(acc[i][j][r]);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int gn = col_base + j * 32;
                if (gn >= g.N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gm = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (gm < g.M) C[(int64_t)gm * g.scm + (int64_t)gn * g.scn] = from_f32<TO>(acc[i][j][r]);
                }
            }
    }
}

// Four consecutive elements p[off .. off+3] (element stride 1) of dtype dt
// as fp32, in one vector load when `vec` (the caller checked 4-element
// alignment), else element by element for the first n (n <= 4) of them.
__device__ __forceinline__ void load4(const void *p, int64_t off, int dt, bool vec, int n, float (&out)[4]) {
    if (dt == DG_F32) {
        const float *q = static_cast<const float *>(p) + off;
        if (vec) {
            const float4 v = *reinterpret_cast<const float4 *>(q);
            out[0] = v.x, out[1] = v.y, out[2] = v.z, out[3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = e < n ? q[e] : 0.0f;
        }
        return;
    }
    const uint16_t *q = static_cast<const uint16_t *>(p) + off;
    uint16_t h[4];
    if (vec) {
        const uint2 v = *reinterpret_cast<const uint2 *>(q);
        h[0] = (uint16_t)v.x, h[1] = (uint16_t)(v.x >> 16), h[2] = (uint16_t)v.y, h[3] = (uint16_t)(v.y >> 16);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = e < n ? q[e] : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = dt == DG_BF16 ? to_f32<BF16>(h[e]) : to_f32<F16>(h[e]);
}

// Per-thread view of the staged tile for the fused epilogue: one 4-column
// group (columns gn0 .. gn0+3 of C, ncols of them inside C) and the uniform
// operands, decided once per tile.
struct EpiRows {
    const float *st;         // staged rows (LDS), row pitch ldn floats
    int ldn, c4, r0, rs;     // this thread's column group in the tile, first row, row step
    int m_row0;              // C row of staged row 0
    int rows;                // staged rows inside C
    int gn0, ncols;
    char *C;                 // C of this product (bytes)
    int c_es;
    bool cvec, rvec, use_r;
    int rmode;               // 16-bit residual requested per pass: 1 bf16, 2 fp16; 0: read at use
    int64_t r_off, b_off;
    float bcol[4];           // per-column bias of the group (0 if none)
    bool row_bias;
};

// Rounds and stores 4 values of one row (dtype OUT), vector store when vec.
template <int OUT>
__device__ __forceinline__ void store4_t(char *p, bool vec, int n, int64_t s, const float (&y)[4]) {
    if constexpr (OUT == DG_F32) {
        float *q = reinterpret_cast<float *>(p);
        if (vec) {
            *reinterpret_cast<float4 *>(q) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < n) q[e * s] = y[e];
        }
    } else {
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = OUT == DG_BF16 ? from_f32<BF16>(y[e]) : from_f32<F16>(y[e]);
        uint16_t *q = reinterpret_cast<uint16_t *>(p);
        if (vec) {
            *reinterpret_cast<uint2 *>(q) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                       (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < n) q[e * s] = h[e];
        }
    }
}

// Issues the 16-bit residual loads (one 8-byte vector per row, rmode 1/2)
// and the per-row bias loads of this thread's RU rows of one pass (rows r0,
// r0 + rs, ...). Nothing waits for them here: the caller stages the
// accumulators meanwhile, so one memory latency per pass is exposed instead
// of one per few rows. An fp32 or unaligned residual (rmode 0) is read where
// it is used (epi_rows), which keeps two words per row here.
template <int RU>
__device__ __forceinline__ void epi_load(const GemmArgs &g, const EpiRows &e, uint32_t (&raw)[RU][2],
                                         float (&br)[RU]) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int row = e.r0 + u * e.rs;
        const bool in = row < e.rows;
        const int gm = e.m_row0 + row;
        raw[u][0] = raw[u][1] = 0u;
        if (in && e.rmode != 0) {
            const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(g.R) + e.r_off +
                                                             (int64_t)gm * g.srm + e.gn0);
            raw[u][0] = v.x, raw[u][1] = v.y;
        }
        br[u] = (in && e.row_bias) ? load_any(g.bias, e.b_off + (int64_t)gm * g.sbias, g.bias_dtype) : 0.0f;
    }
}

// The staged rows of one pass through act(alpha*x + beta*R + bias), for one
// activation (so the per-element work has no branches: an absent residual or
// bias enters as +0, which changes at most the sign of a zero result). The
// output dtype is a uniform branch per row: one copy of the row code per
// activation keeps the kernel's code small, and the tile's tail runs once
// per tile, out of the instruction cache.
template <int ACT, int RU>
__device__ __forceinline__ void epi_rows(const GemmArgs &g, const EpiRows &e, const uint32_t (&raw)[RU][2],
                                         const float (&br)[RU]) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int row = e.r0 + u * e.rs;
        if (row >= e.rows) continue;
        float rv[4];
        if (e.rmode != 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint16_t h = (uint16_t)(raw[u][k >> 1] >> (16 * (k & 1)));
                rv[k] = e.rmode == 1 ? to_f32<BF16>(h) : to_f32<F16>(h);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) rv[k] = 0.0f;
            if (e.use_r) {
                const int64_t off = e.r_off + (int64_t)(e.m_row0 + row) * g.srm;
                if (g.srn == 1) {
                    load4(g.R, off + e.gn0, g.r_dtype, e.rvec, e.ncols, rv);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (k < e.ncols) rv[k] = load_any(g.R, off + (int64_t)(e.gn0 + k) * g.srn, g.r_dtype);
                }
            }
        }
        const float4 v = *reinterpret_cast<const float4 *>(e.st + row * e.ldn + e.c4);
        const float x[4] = {v.x, v.y, v.z, v.w};
        float y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float t = __builtin_fmaf(g.beta, rv[k], g.alpha * x[k]) + (e.bcol[k] + br[u]);
            if constexpr (ACT == DG_ACT_RELU) t = t < 0.0f ? 0.0f : t;
            if constexpr (ACT == DG_ACT_GELU) t = activate(t, DG_ACT_GELU);
            if constexpr (ACT == kActGelu16) t = gelu_16(t);
            y[k] = t;
        }
        char *cp = e.C + ((int64_t)(e.m_row0 + row) * g.scm + (int64_t)e.gn0 * g.scn) * e.c_es;
        if (g.out_dtype == DG_BF16) store4_t<DG_BF16>(cp, e.cvec, e.ncols, g.scn, y);
        else if (g.out_dtype == DG_F16) store4_t<DG_F16>(cp, e.cvec, e.ncols, g.scn, y);
        else store4_t<DG_F32>(cp, e.cvec, e.ncols, g.scn, y);
    }
}

// The fused epilogue without LDS, for an interior tile whose epilogue needs
// nothing from other lanes: no residual (beta == 0), bias absent or one per
// column, any activation (each acts on one element). In the accumulator
// layout every register of lane l in fragment column j lies in column
// col_base + 32j, so the lane loads one bias value per fragment column and
// stores each element straight from its register, as the plain store does
// (measured faster than staging the tile for whole-row writes). Same
// arithmetic as epi_rows, absent terms as +0. GELU is a template argument
// (DG_ACT_GELU for fp32 outputs, kActGelu16 for 16-bit ones, as in
// epi_rows); none and ReLU share one instantiation.
template <typename TO, int GELU, int FM, int FN>
__device__ __forceinline__ void epi_direct_t(const GemmArgs &g, const EpiRows &e, const f32x16 (&acc)[FM][FN],
                                             int row_base, int col_base) {
    typename TO::storage *C = reinterpret_cast<typename TO::storage *>(e.C);  // this product's C
    const bool relu = g.act == DG_ACT_RELU;
    float bc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        bc[j] = g.bias ? load_any(g.bias, e.b_off + (int64_t)(col_base + j * 32) * g.sbias, g.bias_dtype) : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t cbase = (int64_t)(col_base + j * 32) * g.scn;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                float t = __builtin_fmaf(g.beta, 0.0f, g.alpha * acc[i][j][r]) + (bc[j] + 0.0f);
                if constexpr (GELU == DG_ACT_GELU) t = activate(t, DG_ACT_GELU);
                else if constexpr (GELU == kActGelu16) t = gelu_16(t);
                else t = (relu && t < 0.0f) ? 0.0f : t;
                C[(int64_t)gm * g.scm + cbase] = from_f32<TO>(t);
            }
        }
}

template <int FM, int FN, bool GELU>
__device__ __forceinline__ void epi_direct(const GemmArgs &g, const EpiRows &e, const f32x16 (&acc)[FM][FN],
                                           int row_base, int col_base) {
    if (GELU && g.act == DG_ACT_GELU) {
        if (g.out_dtype == DG_BF16) epi_direct_t<BF16, kActGelu16, FM, FN>(g, e, acc, row_base, col_base);
        else if (g.out_dtype == DG_F16) epi_direct_t<F16, kActGelu16, FM, FN>(g, e, acc, row_base, col_base);
        else epi_direct_t<F32, DG_ACT_GELU, FM, FN>(g, e, acc, row_base, col_base);
        return;
    }
    if (g.out_dtype == DG_BF16) epi_direct_t<BF16, 0, FM, FN>(g, e, acc, row_base, col_base);
    else if (g.out_dtype == DG_F16) epi_direct_t<F16, 0, FM, FN>(g, e, acc, row_base, col_base);
    else epi_direct_t<F32, 0, FM, FN>(g, e, acc, row_base, col_base);
}

// The same tile through the fused epilogue, staged through LDS. The tile is
// written to LDS (fp32, rows padded by 4 floats) in passes of whole 32-row
// fragment blocks. Each thread then owns one 4-column group of the tile
// (T is a multiple of BN/4) and walks its rows of each pass, RU at a time: a
// per-column bias is loaded once per tile, the pass's residual rows are
// requested before the staging (epi_load), and a row's 4 elements of C and of
// the residual move as one vector when the layout allows. `st` is the
// kernel's LDS (CAP bytes, free: the K loop is done).
template <int BM, int BN, int WM, int WN, int FM, int FN, int CAP, bool DIRECT_GELU = true>
__device__ __forceinline__ void store_epi(const GemmArgs &g, const WorkItem &w, const f32x16 (&acc)[FM][FN],
                                          float *st, int m0, int n0) {
    constexpr int T = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int LDN = BN + 4;
    constexpr int Q = BN / 4;  // 4-column groups per row
    static_assert(T % Q == 0, "every thread keeps one column group");
    constexpr int RS = T / Q;  // rows between a thread's rows
    constexpr int FIT = CAP / 4 / LDN;
    // Rows per pass: whole 32-row blocks that fit in LDS (PRN). When a
    // residual or per-row bias is read, at most RU = 8 rows per thread (PRL),
    // which bounds the registers holding the pass's requested rows; the rows
    // of a pass are then handled in chunks of RU rows per thread.
    constexpr int PRN = FIT >= BM ? BM : (FIT / 32) * 32;
    static_assert(PRN >= 32, "LDS too small to stage 32 rows of the tile");
    constexpr int RU = 8;
    constexpr int PRC = (RU * RS) / 32 * 32;
    constexpr int PRL = PRN < PRC ? PRN : (PRC >= 32 ? PRC : 32);
    static_assert(PRL <= RU * RS, "a loading pass fits one chunk of rows");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    EpiRows e;
    e.st = st;
    e.ldn = LDN;
    e.c4 = (tid % Q) * 4;
    e.r0 = tid / Q;
    e.rs = RS;
    e.gn0 = n0 + e.c4;
    e.ncols = min(4, g.N - e.gn0);
    e.c_es = g.out_dtype == DG_F32 ? 4 : 2;
    e.C = static_cast<char *>(g.C) + (int64_t)w.prod * g.bsc * e.c_es;
    e.use_r = g.beta != 0.0f;
    e.r_off = (int64_t)w.prod * g.bsr;
    e.b_off = (int64_t)w.prod * g.bsbias;
    e.row_bias = g.bias != nullptr && g.bias_per_row;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        e.bcol[k] = (g.bias != nullptr && !g.bias_per_row && k < e.ncols)
                        ? load_any(g.bias, e.b_off + (int64_t)(e.gn0 + k) * g.sbias, g.bias_dtype)
                        : 0.0f;
    const int r_es = g.r_dtype == DG_F32 ? 4 : 2;
    e.cvec = e.ncols == 4 && g.scn == 1 && g.scm % 4 == 0 &&
             ((uintptr_t)(e.C + (int64_t)e.gn0 * e.c_es) % (uintptr_t)(4 * e.c_es)) == 0;
    e.rvec = e.ncols == 4 && e.use_r && g.srn == 1 && g.srm % 4 == 0 &&
             ((uintptr_t)g.R + (uintptr_t)((e.r_off + e.gn0) * r_es)) % (uintptr_t)(4 * r_es) == 0;
    e.rmode = (!e.rvec || r_es == 4) ? 0 : (g.r_dtype == DG_BF16 ? 1 : 2);
    // DIRECT_GELU false keeps GELU on the staged path (a kernel whose
    // registers would not hold the direct path's GELU without spilling).
    if (!e.use_r && !e.row_bias && (DIRECT_GELU || g.act != DG_ACT_GELU) && m0 + BM <= g.M && n0 + BN <= g.N) {
        epi_direct<FM, FN, DIRECT_GELU>(g, e, acc, m0 + wm * WTM + 4 * (lane >> 5), n0 + wn * WTN + (lane & 31));
        return;
    }
    // The pass loop; the pass size is a compile-time constant, so the staging
    // of each fragment block resolves statically.
    auto passes = [&](auto pr_tag) {
        constexpr int PR = decltype(pr_tag)::value;
        uint32_t raw[RU][2];
        float br[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) raw[u][0] = raw[u][1] = 0u, br[u] = 0.0f;
#pragma unroll 1
        for (int p0 = 0; p0 < BM; p0 += PR) {
            e.m_row0 = m0 + p0;
            // Rows of this pass inside the tile and inside C. The tile bound
            // matters when PR does not divide BM: the last pass then holds
            // fewer than PR rows, and the rows past the tile belong to the
            // next tile's workgroup.
            e.rows = min(min(PR, BM - p0), g.M - m0 - p0);
            epi_load<RU>(g, e, raw, br);
            __syncthreads();  // the previous pass (or the K loop) is done with the LDS
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int rb = wm * WTM + i * 32 - p0;  // block's first row within this pass
                if (rb < 0 || rb >= PR) continue;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = wn * WTN + j * 32 + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        st[(rb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * LDN + col] = acc[i][j][r];
                }
            }
            __syncthreads();
            if (e.ncols <= 0) continue;
            // The pass in chunks of RU rows per thread (one chunk when rows
            // were requested ahead: PRL <= RU * RS).
#pragma unroll 1
            for (int c = 0; c < PR; c += RU * RS) {
                EpiRows ec = e;
                ec.r0 = e.r0 + c;
                if (g.act == DG_ACT_GELU && g.out_dtype == DG_F32) epi_rows<DG_ACT_GELU, RU>(g, ec, raw, br);
                else if (g.act == DG_ACT_GELU) epi_rows<kActGelu16, RU>(g, ec, raw, br);
                else if (g.act == DG_ACT_RELU) epi_rows<DG_ACT_RELU, RU>(g, ec, raw, br);
                else epi_rows<DG_ACT_NONE, RU>(g, ec, raw, br);
            }
        }
    };
    // Every epilogue stages PRL rows per pass (a divisor of BM; 64 on the
    // 128- and 256-row tiles). An earlier variant staged PRN = 96 rows per pass on
    // 256x256 and 128x128 tiles and bounded a pass's rows by C only, not by
    // the tile: its last pass (rows 192..287 of a 256-row tile, 96..191 of a
    // 128-row tile) wrote stale staged rows into the first 32 or 64 rows of
    // the next tile down, racing with that tile's own workgroup. That is the
    // 15/128 of C it got wrong at 4096^3 (15 of 16 tile rows spill 32 rows
    // each) and the run-to-run variation at 128x128. The bound above closes
    // it for any pass size.
    static_assert(BM % PRL == 0, "whole passes: the pass loop covers the tile exactly");
    passes(std::integral_constant<int, PRL>{});
}

// ---- split-K -------------------------------------------------------------------
// The K loop is cut into g.splits ranges, each run by its own workgroup
// (more workgroups in flight when a problem has few output tiles; latency
// is hidden by having many programs in flight, "Triton：04 Matmul、Autotune 与
// PyTorch 集成"). Each workgroup stores its fp32 partial tile to the
// workspace and exits; a second kernel (gemm_split_reduce, same tile shape
// and thread layout) adds the partials of a tile in range order 0, 1, ...,
// S-1 -- so the result does not depend on which range finished first -- and
// runs the epilogue. The kernel boundary makes the partials visible to the
// reducer on every XCD. (Doing the reduction in the last-arriving workgroup
// instead needs device-scope release/acquire fences per workgroup, which
// write back and invalidate the XCD's whole L2; measured, that made a
// 1024^3 split 8x slower than no split.)
//
// Workspace layout of a partial: float4 v of thread t at [v * T + t], v over
// (block i, block j, quarter q) = registers 4q..4q+3 of acc[i][j]; the S
// partials of one (product, tile) slot are consecutive.
template <int FM, int FN, int T>
__device__ __forceinline__ void split_store(const GemmArgs &g, const WorkItem &w, const f32x16 (&acc)[FM][FN]) {
    constexpr int V = FM * FN * 4;
    float4 *mine = reinterpret_cast<float4 *>(g.ws) + ((int64_t)w.slot * g.splits + w.split) * (V * T);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mine[((i * FN + j) * 4 + q) * T + threadIdx.x] =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
}

// How a kernel instantiation finishes its tile. Each MFMA kernel is compiled
// once per mode and the launcher picks the instantiation from the
// arguments: the fused epilogue's registers and code would otherwise change
// how the compiler schedules the K loop of the plain kernel (measured: 9%
// slower at 4096^3).
enum EpiMode : int { EM_STORE = 0, EM_FUSED = 1, EM_SPLIT = 2, EM_STREAMK = 3 };

// Plain stores straight from the accumulator registers.
template <int BM, int BN, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void write_plain(const GemmArgs &g, const WorkItem &w, const f32x16 (&acc)[FM][FN],
                                            int m0, int n0) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row_base = m0 + (wave / WN) * WTM + 4 * (lane >> 5);
    const int col_base = n0 + (wave % WN) * WTN + (lane & 31);
    const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;
    const int64_t c_off = (int64_t)w.prod * g.bsc;
    if (g.out_dtype == DG_BF16) store_acc<BF16, FM, FN>(g, c_off, acc, row_base, col_base, interior);
    else if (g.out_dtype == DG_F16) store_acc<F16, FM, FN>(g, c_off, acc, row_base, col_base, interior);
    else store_acc<F32, FM, FN>(g, c_off, acc, row_base, col_base, interior);
}

// Either epilogue, chosen at run time (the split-K reduction kernel).
template <int BM, int BN, int WM, int WN, int FM, int FN, int CAP>
__device__ __forceinline__ void write_tile(const GemmArgs &g, const WorkItem &w, const f32x16 (&acc)[FM][FN],
                                           float *st, int m0, int n0) {
    if (g.epi) store_epi<BM, BN, WM, WN, FM, FN, CAP>(g, w, acc, st, m0, n0);
    else write_plain<BM, BN, WM, WN, FM, FN>(g, w, acc, m0, n0);
}

// The end of an MFMA kernel in mode EM.
template <int EM, int BM, int BN, int WM, int WN, int FM, int FN, int CAP, bool DIRECT_GELU = true>
__device__ __forceinline__ void finish_tile(const GemmArgs &g, const WorkItem &w, const f32x16 (&acc)[FM][FN],
                                            float *st, int m0, int n0) {
    if constexpr (EM == EM_SPLIT) split_store<FM, FN, WM * WN * 64>(g, w, acc);  // gemm_split_reduce finishes it
    else if constexpr (EM == EM_FUSED) store_epi<BM, BN, WM, WN, FM, FN, CAP, DIRECT_GELU>(g, w, acc, st, m0, n0);
    else write_plain<BM, BN, WM, WN, FM, FN>(g, w, acc, m0, n0);
}

// Buffer resources (raw, 32-bit data format) for the buffer load and store
// builtins.
constexpr int kOobOffset = (int)0x80000000;  // buffer offset >= num_records: loads zero
constexpr int kNumRecords = 0x7fffffff;
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, 32-bit data format

// s_waitcnt vmcnt(0) (expcnt/lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- stream-K ------------------------------------------------------------------
// A persistent grid of G workgroups (at most one per CU, so all are resident
// at once) shares out the tiles' K steps evenly instead of whole tiles, so a
// tile count just past a multiple of G does not cost a whole extra round of
// tiles (the wave quantisation that shapes needing their own configs run
// into, "Triton：04 Matmul、Autotune 与 PyTorch 集成"). Rank r of G:
//  1. computes whole tiles sk_tiles + r, sk_tiles + r + G, ... (all K);
//  2. takes its share of the S = sk_tiles * sk_iters K steps of the first
//     sk_tiles tiles, numbered tile-major: ranks below S % G take S / G + 1
//     consecutive steps, the others S / G (S < 2^31, checked on the host).
//     The host shares the partial last round together with one whole round
//     (so every rank takes one to two tiles' steps and a tile has at most
//     three pieces), and launches at most two ranks per tile when there are
//     fewer tiles than CUs. The range is split at
//     tile boundaries into pieces. A piece that starts inside its tile
//     (only a rank's first piece can) stores its fp32 partial tile in slot r
//     and then raises flag r. A piece that starts at the tile's first K step
//     belongs to the tile's owner: it adds the partials of the ranks that
//     cover the rest of the tile, in rank order (= K order, so the result
//     does not depend on timing), and runs the epilogue.
// An owner waits only on higher ranks' first pieces, which wait on nothing,
// so the grid cannot deadlock while all its workgroups are resident; the wait
// is still bounded (a partial that never arrives leaves NaN in the tile).
// Partials and flags cross XCDs: they are written and read with agent-scope
// atomic accesses, which bypass the non-coherent caches line by line, and
// the flag is stored only after the partial's stores have completed. This
// avoids the release/acquire fences, which write back or invalidate a
// whole L2.
//
// Workspace: G 8-byte flags (padded to 256 bytes), then G partial tiles in
// split_store's layout. A flag holds the launch's epoch in its low word and
// the epoch's complement in its high word, so flags left by earlier launches
// (or other data) never read as raised.
constexpr int kSkSpinLimit = 1 << 20;
constexpr int kSc1 = 16;  // buffer cache-policy operand: the sc1 (agent-scope coherent) bit

// Bit casts through a by-value scalar: applied directly to a vector element
// (acc[i][j][r], d[c]), __builtin_bit_cast reads element 0 whatever the index
// (seen with this compiler), so elements always pass through these.
__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// (product, tile) of stream-K tile number t: products outermost, the
// group-major order within a product.
__device__ __forceinline__ WorkItem sk_tile(int t, const GemmArgs &g) {
    const int tiles = g.grid_m * g.grid_n;
    WorkItem w;
    w.prod = t / tiles;
    w.split = 0;
    group_major(t - w.prod * tiles, g.grid_m, g.grid_n, g.group_m, w.pm, w.pn);
    w.slot = w.prod * tiles + w.pm * g.grid_n + w.pn;
    return w;
}

template <int BM, int BN, int BK, int WM, int WN, int FM, int FN, int CAP, typename Body>
__device__ __forceinline__ void stream_k(const GemmArgs &g, float *st, Body &body) {
    constexpr int T = WM * WN * 64;
    constexpr int V = FM * FN * 4;  // float4s per thread in a partial
    const int G = gridDim.x;
    const int r = (g.xcd_remap && g.num_xcd > 1) ? xcd_rank(blockIdx.x, G, g.num_xcd) : (int)blockIdx.x;
    const int total = g.grid_m * g.grid_n * g.batch;
    const int I = g.sk_iters;
    uint64_t *flags = reinterpret_cast<uint64_t *>(g.ws);
    float *parts = reinterpret_cast<float *>(reinterpret_cast<char *>(g.ws) + sk_flag_bytes(G));
    const uint64_t mark = ((uint64_t)(~g.sk_epoch) << 32) | g.sk_epoch;
    // One call site for the tile body: whole tiles first, then the pieces.
    const int base = g.sk_base, extra = g.sk_extra;  // S / G, S % G
    auto share_begin = [&](int q) { return q * base + min(q, extra); };
    int it = share_begin(r);
    const int it1 = share_begin(r + 1);
    int next_whole = g.sk_tiles + r;
    for (bool first = true;; first = false) {
        int t, kb, ke;
        bool whole;
        if (next_whole < total) {
            t = next_whole;
            kb = 0;
            ke = I;
            whole = true;
            next_whole += G;
        } else if (it < it1) {
            t = it / I;
            kb = it - t * I;            // first K step of the piece
            ke = min(I, it1 - t * I);   // one past its last
            whole = false;
            it = t * I + ke;
        } else {
            break;
        }
        if (!first) __syncthreads();  // the previous tile is done with the LDS
        const WorkItem w = sk_tile(t, g);
        f32x16 acc[FM][FN];
        body(w, kb * BK, min(g.K, ke * BK) - kb * BK, acc);
        // Partials move as 16-byte buffer accesses with the agent-scope
        // coherence bit (sc1): float4 v of thread t at byte (v * T + t) * 16 of
        // the rank's slot, the register offset fixed and the slice offset a
        // scalar, so no per-access address registers.
        const int voff = threadIdx.x * 16;
        if (kb > 0) {
            const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
                parts + (int64_t)r * (V * T * 4), 0, V * T * 16, kRsrcWord3);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        u32x4 d;
#pragma unroll
                        for (int c = 0; c < 4; ++c) d[c] = f32_bits(acc[i][j][4 * q + c]);
                        __builtin_amdgcn_raw_buffer_store_b128(d, mine, voff, ((i * FN + j) * 4 + q) * T * 16,
                                                               kSc1);
                    }
            wait_vmcnt0();  // this thread's stores have completed
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_store(flags + r, mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        if (!whole) {
            const int tile_end = (t + 1) * I;
            for (int q = r + 1; q < G; ++q) {
                const int q0 = share_begin(q);
                if (q0 >= tile_end) break;
                if (share_begin(q + 1) == q0) continue;  // rank q has no steps
                // Each wave watches the flag itself (lane 0) and reads the
                // partial after seeing it raised.
                int spins = 0;
                if ((threadIdx.x & 63) == 0)
                    while (__hip_atomic_load(flags + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != mark &&
                           ++spins < kSkSpinLimit)
                        __builtin_amdgcn_s_sleep(2);
                const bool lost = __builtin_amdgcn_readfirstlane(spins) >= kSkSpinLimit;
                const __amdgpu_buffer_rsrc_t theirs = __builtin_amdgcn_make_buffer_rsrc(
                    parts + (int64_t)q * (V * T * 4), 0, V * T * 16, kRsrcWord3);
                // CH float4s requested together (the whole partial of a small
                // tile, 16 at a time of a large one), then added.
                constexpr int CH = V < 16 ? V : 16;
#pragma unroll
                for (int v0 = 0; v0 < V; v0 += CH) {
                    u32x4 d[CH];
#pragma unroll
                    for (int u = 0; u < CH; ++u)
                        d[u] = __builtin_amdgcn_raw_buffer_load_b128(theirs, voff, (v0 + u) * T * 16, kSc1);
#pragma unroll
                    for (int u = 0; u < CH; ++u) {
                        const int v = v0 + u, i = v / (FN * 4), j = (v / 4) % FN, q4 = v % 4;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            acc[i][j][4 * q4 + c] =
                                lost ? __builtin_nanf("") : acc[i][j][4 * q4 + c] + bits_f32(d[u][c]);
                    }
                }
            }
        }
        write_tile<BM, BN, WM, WN, FM, FN, CAP>(g, w, acc, st, w.pm * BM, w.pn * BN);
    }
}

// The work of one launch: one tile (or K range) per workgroup, or stream-K.
// body(w, k_begin, kl, acc) computes tile w over k in [k_begin, k_begin + kl).
template <int EM, int BM, int BN, int BK, int WM, int WN, int FM, int FN, int CAP, typename Body>
__device__ __forceinline__ void run_tiles(const GemmArgs &g, float *st, Body &&body) {
    if constexpr (EM == EM_STREAMK) {
        stream_k<BM, BN, BK, WM, WN, FM, FN, CAP>(g, st, body);
    } else {
        const WorkItem w = work_item(blockIdx.x, g);
        const int k_begin = w.split * g.k_chunk;
        const int kl = min(g.K - k_begin, g.k_chunk);  // this workgroup's K range
        f32x16 acc[FM][FN];
        body(w, k_begin, kl, acc);
        // Epilogue: fp32 accumulators -> C's dtype, masked to C's view.
        finish_tile<EM, BM, BN, WM, WN, FM, FN, CAP>(g, w, acc, st, w.pm * BM, w.pn * BN);
    }
}

// One output tile of the register-staged kernel: WM x WN waves, each owning
// a (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks; acc receives the tile's
// sum over k in [k_begin, k_begin + kl). LDK is the LDS row pitch in
// elements: +16 B breaks the bank pattern of 128 B rows.
template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB>
__device__ __forceinline__ void mfma_reg_tile(const GemmArgs &g, const WorkItem &w, int k_begin, int kl,
                                              uint16_t (&lds)[2][(BM + BN) * (BK + 8)],
                                              f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
    constexpr int T = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LDK = BK == 32 ? 32 : BK + 8;  // row pitch (elements), see reg_lds_off
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 16 == 0, "tile shape");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "8-row blocks");
    static_assert(BK == 32 || BK == 64, "reg_lds_off layouts");

    const int m0 = w.pm * BM, n0 = w.pn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // P register sets for the global loads: slice kt+P-1 is requested at
    // step kt and written to LDS at step kt+P-2, so P-1 steps of products
    // cover a load's latency. Small tiles do little work per step and take
    // 4 sets; 128x128 and larger keep 2 (their registers are the limit).
    // Small tiles whose operands are both k-contiguous (any alignment) run
    // the branch-free loop below (KuStream): the K tail is loaded like every
    // other slice, 16 bytes per chunk, instead of element by element behind
    // a branch, which made its step wait a full memory latency. (The host
    // sends such problems here only when K >= 8.)
    constexpr bool DEEP = LA == LD_KU && LB == LD_KU && BM * BN < 128 * 128;
    constexpr int P = BM * BN < 128 * 128 ? 4 : 2;
    // With P = 2 one set serves both roles (requested at the top of a step,
    // written at its end), as the register budget of the large tiles needs.
    constexpr int NSET = (P == 2 || DEEP) ? 1 : P;
    TileLoader<BM, BK, LDK, T, LA> la[NSET];
    TileLoader<BN, BK, LDK, T, LB> lb[NSET];
    const uint16_t *A = static_cast<const uint16_t *>(g.A) + (int64_t)w.prod * g.bsa;
    const uint16_t *B = static_cast<const uint16_t *>(g.B) + (int64_t)w.prod * g.bsb;
#pragma unroll
    for (int p = 0; p < NSET; ++p) {
        la[p].base = A + (int64_t)m0 * g.sam + (int64_t)k_begin * g.sak;
        la[p].srow = g.sam;
        la[p].sk = g.sak;
        la[p].rows_valid = min(BM, g.M - m0);
        la[p].K = kl;
        lb[p].base = B + (int64_t)n0 * g.sbn + (int64_t)k_begin * g.sbk;
        lb[p].srow = g.sbn;
        lb[p].sk = g.sbk;
        lb[p].rows_valid = min(BN, g.N - n0);
        lb[p].K = kl;
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (kl + BK - 1) / BK;
    // Slices [0, n_fast) take the branch-free loads: wholly inside K.
    const int n_fast = kl / BK;

#pragma unroll
    for (int p = 0; p + 1 < P; ++p) {
        if (!DEEP && p < nk) {
            if ((p + 1) * BK <= kl) {  // p < n_fast
                la[p % NSET].template load<true>(tid, p * BK);
                lb[p % NSET].template load<true>(tid, p * BK);
            } else {
                la[p % NSET].load(tid, p * BK);
                lb[p % NSET].load(tid, p * BK);
            }
        }
    }
    if (!DEEP && nk > 0) {
        la[0].store(tid, lds[0]);
        lb[0].store(tid, lds[0] + BM * LDK);
        __syncthreads();
    }

    // LDS offsets (elements) of this lane's fragment rows. BK 32: the row
    // part, and the permuted chunk of each k-substep (bits 2-3 of the row do
    // not change from one 32-row block to the next).
    const int a_row = (wm * WTM + (lane & 31)) * LDK + (BK == 32 ? 0 : (lane >> 5) * 8);
    const int b_row = (BM + wn * WTN + (lane & 31)) * LDK + (BK == 32 ? 0 : (lane >> 5) * 8);
    int a_ch[2] = {0, 0}, b_ch[2] = {0, 0};
    if constexpr (BK == 32) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            a_ch[kk] = reg_lds_off<BK, LDK>(wm * WTM + (lane & 31), (lane >> 5) * 8 + 16 * kk) -
                       (wm * WTM + (lane & 31)) * LDK;
            b_ch[kk] = reg_lds_off<BK, LDK>(BM + wn * WTN + (lane & 31), (lane >> 5) * 8 + 16 * kk) -
                       (BM + wn * WTN + (lane & 31)) * LDK;
        }
    }

    // Step kt: request slice kt+P-1 into set (kt+P-1) % P, multiply slice kt
    // (LDS buffer kt & 1), write slice kt+1 from set (kt+1) % P into the other
    // buffer (read in step kt-1, before the last barrier). Steps run P at a
    // time so the set and buffer indices are compile-time (P is even).
    static_assert(P % 2 == 0, "buffer parity follows the step within a group");
    auto multiply = [&](int u) {
        const uint16_t *s = lds[u & 1];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(s + a_row + i * 32 * LDK + (BK == 32 ? a_ch[kk] : kk * 16));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const u32x4 *>(s + b_row + j * 32 * LDK + (BK == 32 ? b_ch[kk] : kk * 16));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<TI>::run(af[i], bf[j], acc[i][j]);
        }
    };
    if constexpr (DEEP) {
        // Slices 0..P-2 into sets 0..P-2, then whole groups of P steps: step
        // kt requests slice kt+P-1 (a clamped dummy past K) and writes slice
        // kt+1 into the other buffer; straight-line code with compile-time
        // set and buffer indices. The last nk - kt0 < P steps load nothing
        // (every slice they need was requested).
        KuStream<BM, BK, LDK, T, P> sa;
        KuStream<BN, BK, LDK, T, P> sb;
        sa.init(la[0].base, g.sam, la[0].rows_valid, kl, tid);
        sb.init(lb[0].base, g.sbn, lb[0].rows_valid, kl, tid);
#pragma unroll
        for (int p = 0; p + 1 < P; ++p) {
            sa.load(p, tid, p * BK);
            sb.load(p, tid, p * BK);
        }
        sa.store(0, tid, lds[0], 0);
        sb.store(0, tid, lds[0] + BM * LDK, 0);
        __syncthreads();
        int kt0 = 0;
        for (; kt0 + P <= nk; kt0 += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int kt = kt0 + u;
                sa.load((u + P - 1) % P, tid, (kt + P - 1) * BK);
                sb.load((u + P - 1) % P, tid, (kt + P - 1) * BK);
                multiply(u);
                sa.store((u + 1) % P, tid, lds[(u & 1) ^ 1], (kt + 1) * BK);
                sb.store((u + 1) % P, tid, lds[(u & 1) ^ 1] + BM * LDK, (kt + 1) * BK);
                __syncthreads();
                // keep each step's work in its step: moved earlier, the
                // stores' arithmetic would wait for loads still in flight
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int kt = kt0 + u;
            if (kt < nk) {
                multiply(u);
                if (kt + 1 < nk) {
                    sa.store((u + 1) % P, tid, lds[(u & 1) ^ 1], (kt + 1) * BK);
                    sb.store((u + 1) % P, tid, lds[(u & 1) ^ 1] + BM * LDK, (kt + 1) * BK);
                }
                __syncthreads();
            }
        }
    } else if constexpr (P == 2) {
        // The large tiles: one register set, requested at the top of a step
        // and written at its end (their registers do not allow more). First
        // the steps whose next slice takes the branch-free loads, then the
        // rest, guarded.
        int kt = 0;
        // LD_GN has no branch-free load (both operands use it or neither).
        if constexpr (LA != LD_GN && BK >= 64)
        for (; kt + 2 <= n_fast; ++kt) {
            la[0].template load<true>(tid, (kt + 1) * BK);
            lb[0].template load<true>(tid, (kt + 1) * BK);
            multiply(kt & 1);
            la[0].store(tid, lds[(kt & 1) ^ 1]);
            lb[0].store(tid, lds[(kt & 1) ^ 1] + BM * LDK);
            __syncthreads();
        }
        for (; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                la[0].load(tid, (kt + 1) * BK);
                lb[0].load(tid, (kt + 1) * BK);
            }
            multiply(cur);
            if (more) {
                la[0].store(tid, lds[cur ^ 1]);
                lb[0].store(tid, lds[cur ^ 1] + BM * LDK);
            }
            __syncthreads();
        }
    } else {
        // Groups whose every step exists and requests a slice below n_fast:
        // straight-line code (no branch between a load and the write of its
        // data), so the compiler waits for each set only when it is written.
        int kt0 = 0;
        for (; kt0 + 2 * P - 2 < n_fast; kt0 += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int kt = kt0 + u;
                la[(u + P - 1) % P].template load<true>(tid, (kt + P - 1) * BK);
                lb[(u + P - 1) % P].template load<true>(tid, (kt + P - 1) * BK);
                multiply(u);
                la[(u + 1) % P].store(tid, lds[(u & 1) ^ 1]);
                lb[(u + 1) % P].store(tid, lds[(u & 1) ^ 1] + BM * LDK);
                __syncthreads();
            }
        }
        // The remaining steps, each guarded (the K tail and the end).
        for (; kt0 < nk; kt0 += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int kt = kt0 + u;
                if (kt >= nk) break;
                if (kt + P - 1 < nk) {
                    const int k0 = (kt + P - 1) * BK;
                    if (k0 + BK <= kl) {  // slice below n_fast
                        la[(u + P - 1) % P].template load<true>(tid, k0);
                        lb[(u + P - 1) % P].template load<true>(tid, k0);
                    } else {
                        la[(u + P - 1) % P].load(tid, k0);
                        lb[(u + P - 1) % P].load(tid, k0);
                    }
                }
                multiply(u);
                if (kt + 1 < nk) {
                    la[(u + 1) % P].store(tid, lds[(u & 1) ^ 1]);
                    lb[(u + 1) % P].store(tid, lds[(u & 1) ^ 1] + BM * LDK);
                }
                __syncthreads();
            }
        }
    }
}

template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int EM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mfma(GemmArgs g) {
    constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][(BM + BN) * (BK + 8)];
    run_tiles<EM, BM, BN, BK, WM, WN, FM, FN, (int)sizeof(lds)>(
        g, reinterpret_cast<float *>(&lds[0][0]), [&](const WorkItem &w, int k_begin, int kl, f32x16(&acc)[FM][FN]) {
            mfma_reg_tile<TI, BM, BN, BK, WM, WN, LA, LB>(g, w, k_begin, kl, lds, acc);
        });
}

// ============================================================================
// gemm_mfma_lds: operands travel global -> LDS directly
// ============================================================================
//
// Each 64-lane buffer_load_dwordx4 ... lds writes 1 KiB of LDS: lane i's 16
// bytes land at M0 + 16*i. The tile layout is chosen by which global chunk
// each lane fetches. A buffer offset past num_records reads as zero, which
// masks rows past M/N and k past K without a branch.
//
// Two LDS tile formats:
//  KTile [ROWS][BK], k contiguous (operand with k stride 1). A 32x32x16
//        fragment row is one ds_read_b128. The eight 16-byte chunks of a
//        128-byte row are XOR-swizzled with the row index, so the 8- and
//        16-lane groups of a ds_read_b128 hit distinct banks.
//  RTile [BK][ROWS], rows contiguous (operand with row stride 1, e.g. a
//        row-major B). Fragments come from ds_read_b64_tr_b16, which
//        transposes within 16-lane groups: lane j of a group receives element
//        (j % 4) of the 4-element rows addressed by lanes 4e + j/4, e = 0..3.
//        Chunks are XOR-swizzled per k-line so the k-lines a fragment read
//        touches fall on distinct banks.

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;


template <int ROWS, int BK>
struct KTile {
    static_assert(BK == 64 || BK == 32, "KTile rows are 128 or 64 bytes");
    static constexpr int CPR = BK / 8;            // 16-byte chunks per row
    static constexpr int RPL = 1024 / (BK * 2);   // rows per 1 KiB wave load
    static constexpr int NLOADS = ROWS / RPL;
    static constexpr int BYTES = ROWS * BK * 2;
    // Chunk permutation of a row. A ds_read_b128 fragment read touches one
    // chunk column of 32 consecutive rows. These permutations were checked
    // on gfx950 with the LDS bank-conflict counter: both give 4 LDS cycles
    // per ds_read_b128 (1 KiB), i.e. no conflict cycles. (For 64-byte rows
    // the permutation ((row >> 1) ^ (row >> 3)) & 3 measured 8 cycles.)
    __device__ static __forceinline__ int swz(int row) {
        if constexpr (BK == 64) return (row & 7) ^ ((row >> 3) & 1);
        else return (row >> 2) & 3;
    }
    // Element (row, k) of the tile that lane `lane` of wave load `b` fetches (k a multiple of 8).
    __device__ static __forceinline__ void src(int b, int lane, int &row, int &k) {
        row = b * RPL + lane / CPR;
        k = ((lane % CPR) ^ swz(row)) * 8;
    }
    // Byte offset in the tile of the 16 bytes holding (row, k..k+7).
    __device__ static __forceinline__ int at(int row, int k) {
        return row * (BK * 2) + (((k >> 3) ^ swz(row)) << 4);
    }
};

template <int ROWS, int BK>
struct RTile {
    static constexpr int CPR = ROWS / 8;          // 16-byte chunks per k-line
    static_assert(CPR >= 8, "RTile needs at least 64 rows");
    static constexpr int KPL = 1024 / (ROWS * 2); // k-lines per 1 KiB wave load
    static_assert(KPL >= 1, "RTile k-line larger than one wave load");
    static constexpr int NLOADS = BK / KPL;
    static constexpr int BYTES = ROWS * BK * 2;
    // A ds_read_b64_tr_b16 fragment read touches 4 consecutive k-lines, 64
    // bytes of each (two 16-lane groups). The permutation moves those 64-byte
    // pieces to distinct 64-byte bank windows: XOR of the chunk index with
    // 4*(k % 4) (k-lines of 256 or 512 bytes), or with 4*((k / 2) % 2)
    // (128-byte k-lines, where k and k+1 already differ by 128 bytes).
    // Measured on gfx950: 2 LDS cycles per 512-byte tr read, no conflict
    // cycles; XOR with 2*(k % 4) measured 4 cycles.
    __device__ static __forceinline__ int swz(int k) {
        if constexpr (CPR >= 16) return 4 * (k & 3);
        else return 4 * ((k >> 1) & 1);
    }
    __device__ static __forceinline__ void src(int b, int lane, int &k, int &row) {
        k = b * KPL + lane / CPR;
        row = ((lane % CPR) ^ swz(k)) * 8;
    }
    // Byte offset of element (k, row); row a multiple of 4 for the 8-byte reads.
    __device__ static __forceinline__ int at(int k, int row) {
        return k * (ROWS * 2) + ((((row >> 3) ^ swz(k))) << 4) + ((row & 7) << 1);
    }
};

// MFMA operand for rows [r0, r0+32) x k [k0, k0+16): lane l receives
// (row r0 + l%32, k = k0 + 8*(l/32) + e), e = 0..7.
template <int ROWS, int BK>
__device__ __forceinline__ u32x4 frag_from_ktile(const char *tile, int r0, int k0, int lane) {
    const int row = r0 + (lane & 31);
    const int k = k0 + ((lane >> 5) << 3);
    return *reinterpret_cast<const u32x4 *>(tile + KTile<ROWS, BK>::at(row, k));
}

template <int ROWS, int BK>
__device__ __forceinline__ u32x4 frag_from_rtile(const char *tile, int r0, int k0, int lane) {
    // Lane i of 16-lane group q addresses the 4-element line (k0 + 8*(q/2) + i/4 [+4],
    // r0 + 16*(q%2) + 4*(i%4)); after the transpose lane j of the group holds
    // rows r0 + 16*(q%2) + j at k = k0 + 8*(q/2) + e.
    const int q = lane >> 4, i = lane & 15;
    const int row = r0 + 16 * (q & 1) + 4 * (i & 3);
    const int k = k0 + 8 * (q >> 1) + (i >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)(tile + RTile<ROWS, BK>::at(k, row)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)(tile + RTile<ROWS, BK>::at(k + 4, row)));
    u32x4 r;
    r.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    r.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    r.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    r.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return r;
}

// Per-operand state of the direct loads: the buffer descriptor (tile origin,
// k = 0), each wave load's per-lane byte offset (or kOobOffset), and the
// k stride in bytes. NW is the number of waves that share the loads.
template <int ROWS, int BK, int MODE, int NW>
struct DirectLoader {
    using KT = KTile<ROWS, BK>;
    using RT = RTile<ROWS, BK>;
    static constexpr int NLOADS = MODE == LD_KC ? KT::NLOADS : RT::NLOADS;
    static constexpr int PER = NLOADS / NW;
    static_assert(NLOADS % NW == 0, "wave loads must split evenly over the waves");

    __amdgpu_buffer_rsrc_t rsrc;
    int voff[PER];
    int kstride_bytes;

    __device__ __forceinline__ void init(const uint16_t *origin, int64_t srow, int64_t sk, int rows_valid,
                                         int wave, int lane) {
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)origin, 0, kNumRecords, kRsrcWord3);
        kstride_bytes = (int)(2 * (MODE == LD_KC ? 1 : sk));
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int b = wave + NW * j;
            int row, k;
            if (MODE == LD_KC) KT::src(b, lane, row, k);
            else RT::src(b, lane, k, row);
            const bool ok = row < rows_valid;
            const int64_t e = MODE == LD_KC ? (int64_t)row * srow + k : (int64_t)k * sk + row;
            voff[j] = ok ? (int)(2 * e) : kOobOffset;
        }
    }

    // Queue the tile of k-slice [k0, k0 + BK) into `tile` (this wave's share).
    // MASK_K = false: the caller knows the slice lies inside K (no k mask).
    template <bool MASK_K = true>
    __device__ __forceinline__ void issue(char *tile, int k0, int K, int wave, int lane) const {
        const bool tail = MASK_K && k0 + BK > K;
        const int soff = k0 * kstride_bytes;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int b = wave + NW * j;
            int vo = voff[j];
            if (tail) {
                int row, k;
                if (MODE == LD_KC) KT::src(b, lane, row, k);
                else RT::src(b, lane, k, row);
                if (k0 + k >= K) vo = kOobOffset;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(tile + b * 1024), 16, vo, soff, 0, 0);
        }
    }

    __device__ __forceinline__ u32x4 frag(const char *tile, int r0, int k0, int lane) const {
        if constexpr (MODE == LD_KC) return frag_from_ktile<ROWS, BK>(tile, r0, k0, lane);
        else return frag_from_rtile<ROWS, BK>(tile, r0, k0, lane);
    }
};

// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this
// wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier of the LDS pipeline. The caller has waited for the loads
// it needs. The LDS reads of this wave are drained (lgkmcnt(0)), so the stage
// they read may be refilled once every wave has passed. Unlike
// __syncthreads() there is no release fence: that would also wait for the
// younger loads still in flight into other stages. The empty asm statements
// keep the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// No instruction may be scheduled across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Instruction-order hints for the scheduler: NM MFMAs, each followed by its
// share of ND LDS reads and NV global loads, in that order. Without them the
// compiler pulls every fragment read down to just before its MFMA (fewest
// live registers) and the MFMA pipe waits on LDS latency.
template <int NM, int ND, int NV, int T = 0>
__device__ __forceinline__ void interleave_mfma() {
    if constexpr (T < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        constexpr int d = (T + 1) * ND / NM - T * ND / NM;
        if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);  // LDS reads
        constexpr int v = (T + 1) * NV / NM - T * NV / NM;
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // global loads
        interleave_mfma<NM, ND, NV, T + 1>();
    }
}

// WM x WN waves; LA/LB are LD_KC or LD_RC; S LDS stages. The host guarantees
// chunk-exact validity: for an LD_KC operand K % 8 == 0, for an LD_RC operand
// its row count (M or N) % 8 == 0, and all byte offsets fit in 31 bits.
//
// Pipeline: slices 0..S-2 are queued before the loop. Step kt waits until its
// own slice has landed (the S-2 younger slices may still be in flight),
// synchronises the workgroup (everyone's copy of slice kt is visible and
// everyone has finished slice kt-1), queues slice kt+S-1 into the buffer slice
// kt-1 used, then multiplies slice kt. Slices past K are queued as
// out-of-range loads (zeros into a free buffer) so that every step issues the
// same number of loads and the wait count stays a constant.
// One output tile of the direct kernel; acc receives the tile's sum over k in
// [k_begin, k_begin + kl). `lds` holds S stages of A_BYTES + B_BYTES.
template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int S>
__device__ __forceinline__ void mfma_lds_tile(const GemmArgs &g, const WorkItem &w, int k_begin, int kl,
                                              char (&lds)[S * (BM + BN) * BK * 2],
                                              f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 16 == 0, "tile shape");
    static_assert(S >= 2, "at least two stages");

    const int m0 = w.pm * BM, n0 = w.pn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // With two waves per SIMD (NW = 8) only waves 0..NW/2-1 issue the global
    // loads. The issue arbiter favours the older wave of each SIMD pair, so
    // those waves run ahead and wait at the barrier; the loads go into their
    // streams, and the younger waves' streams hold only MFMAs and LDS reads.
    // (Measured: the older waves wait ~40 % of the loop at the barrier, the
    // younger ~4 %; moving the loads to the older waves gains 4-6 % on
    // 8192x14336x4096 at BK 64 and is neutral at 4096^3; moving them to the
    // younger waves loses 10-15 %.)
    constexpr int NLW = NW >= 8 ? NW / 2 : NW;
    using LoaderA = DirectLoader<BM, BK, LA, NLW>;
    using LoaderB = DirectLoader<BN, BK, LB, NLW>;
    const bool loader = NLW == NW || wave < NLW;
    constexpr int LOADS_PER_SLICE = LoaderA::PER + LoaderB::PER;  // per loading wave
    LoaderA la;
    LoaderB lb;
    la.init(static_cast<const uint16_t *>(g.A) + (int64_t)w.prod * g.bsa + (int64_t)m0 * g.sam +
                (int64_t)k_begin * g.sak,
            g.sam, g.sak, min(BM, g.M - m0), loader ? wave : 0, lane);
    lb.init(static_cast<const uint16_t *>(g.B) + (int64_t)w.prod * g.bsb + (int64_t)n0 * g.sbn +
                (int64_t)k_begin * g.sbk,
            g.sbn, g.sbk, min(BN, g.N - n0), loader ? wave : 0, lane);

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (kl + BK - 1) / BK;
    constexpr int KSUB = BK / 16;  // MFMA k-substeps per slice
    // Fragment registers, double-buffered across k-substeps: set (kk & 1)
    // holds substep kk while the other set is being filled.
    u32x4 af[2][FM], bf[2][FN];
    // Fetch order follows the MFMA order below (B fragments are all used by
    // the first row of MFMAs, A fragments one row at a time).
    auto fetch = [&](const char *stage, int kk, int set) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[set][j] = lb.frag(stage + A_BYTES, wn * WTN + j * 32, kk * 16, lane);
#pragma unroll
        for (int i = 0; i < FM; ++i) af[set][i] = la.frag(stage, wm * WTM + i * 32, kk * 16, lane);
    };
    if (nk > 0) {
#pragma unroll
        for (int s = 0; s < S - 1; ++s) {
            if (loader) {
                la.issue(lds + s * STAGE, s * BK, kl, wave, lane);
                lb.issue(lds + s * STAGE + A_BYTES, s * BK, kl, wave, lane);
            }
        }
        wait_vmcnt<(S - 2) * LOADS_PER_SLICE>();
        stage_barrier();
        fetch(lds, 0, 0);
    }

    // One K step over slice kt (in stage `cur`), fragments of its substep 0
    // already in registers:
    //  - queue slice kt+S-1 into `fill` (the stage slice kt-1 used: every
    //    wave finished reading it before the previous barrier);
    //  - for each substep, fetch the next substep's fragments, then issue
    //    this substep's MFMAs;
    //  - before the last substep, wait for slice kt+1 (this wave's loads),
    //    synchronise, and fetch substep 0 of slice kt+1 from `next`, so the
    //    MFMA pipe stays fed across the barrier.
    // Slices past K are queued as out-of-range loads (zeros into a free
    // stage) so every step issues the same number of loads and the wait
    // count is a constant. `cur` never overlaps `fill`; saying so (restrict)
    // keeps the compiler from making the reads of `cur` wait for those loads.
    constexpr int NMFMA = FM * FN;  // MFMAs per substep
    constexpr int NREAD = FM * (LA == LD_KC ? 1 : 2) + FN * (LB == LD_KC ? 1 : 2);  // LDS reads per fetch
    auto mfmas = [&](int set, int from, int to) {
#pragma unroll
        for (int t = from; t < to; ++t) acc[t / FN][t % FN] = Mfma<TI>::run(af[set][t / FN], bf[set][t % FN], acc[t / FN][t % FN]);
    };
    auto step = [&](auto mask_k, char *fill, const char *__restrict__ cur, const char *next, int kt) {
        constexpr bool MASK_K = decltype(mask_k)::value;
        if (loader) {
            la.template issue<MASK_K>(fill, (kt + S - 1) * BK, kl, wave, lane);
            lb.template issue<MASK_K>(fill + A_BYTES, (kt + S - 1) * BK, kl, wave, lane);
        }
#pragma unroll
        for (int kk = 0; kk + 1 < KSUB; ++kk) {
            fetch(cur, kk + 1, (kk & 1) ^ 1);
            mfmas(kk & 1, 0, NMFMA);
        }
        // last substep: half of its MFMAs cover the wait and the barrier
        constexpr int LAST = (KSUB - 1) & 1;
        mfmas(LAST, 0, NMFMA / 2);
        // the slice's global loads go out with the first substep's MFMAs
        interleave_mfma<NMFMA, NREAD, LOADS_PER_SLICE>();
        interleave_mfma<NMFMA * (KSUB - 2), NREAD * (KSUB - 2), 0>();
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA / 2, 0);
        sched_fence();
        wait_vmcnt<(S - 2) * LOADS_PER_SLICE>();
        stage_barrier();
        sched_fence();
        fetch(next, 0, LAST ^ 1);
        mfmas(LAST, NMFMA / 2, NMFMA);
        interleave_mfma<NMFMA - NMFMA / 2, NREAD, 0>();
        sched_fence();
    };
    static_assert(KSUB % 2 == 0, "substep 0 of every slice uses fragment set 0");
    // Slice kt lives in stage kt % S. Steps whose prefetched slice kt+S-1 lies
    // inside K (kt < n_full) need no k mask; they run S at a time, so every
    // stage address is a compile-time offset and the loop carries no address
    // or mask arithmetic. The last steps (at most S-1 + S-1 of them) run with
    // the stage chosen at run time and the masked loads.
    const int n_full = max(0, min(nk, kl / BK - (S - 1)));
    int kt = 0;
    for (; kt + S <= n_full; kt += S) {
#pragma unroll
        for (int u = 0; u < S; ++u)
            step(std::false_type{}, lds + ((u + S - 1) % S) * STAGE, lds + u * STAGE, lds + ((u + 1) % S) * STAGE,
                 kt + u);
    }
    for (; kt < nk; ++kt) {
        const int cur = kt % S;
        const int fill = cur == 0 ? S - 1 : cur - 1;  // stage of slice kt-1 == slice kt+S-1
        const int next = cur + 1 == S ? 0 : cur + 1;
        step(std::true_type{}, lds + fill * STAGE, lds + cur * STAGE, lds + next * STAGE, kt);
    }
    wait_vmcnt<0>();  // the out-of-range tail loads must land before the workgroup can exit
}

template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int S, int EM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mfma_lds(GemmArgs g) {
    constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
    // One LDS object only: the compiler proves the fragment reads independent
    // of the in-flight LDS loads per object, and a second __shared__ variable
    // makes it wait for every load before each read. The epilogue reuses this
    // LDS once the K loop is done.
    __shared__ __attribute__((aligned(1024))) char lds[S * (BM + BN) * BK * 2];
    run_tiles<EM, BM, BN, BK, WM, WN, FM, FN, (int)sizeof(lds)>(
        g, reinterpret_cast<float *>(lds), [&](const WorkItem &w, int k_begin, int kl, f32x16(&acc)[FM][FN]) {
            mfma_lds_tile<TI, BM, BN, BK, WM, WN, LA, LB, S>(g, w, k_begin, kl, lds, acc);
        });
}

// ============================================================================
// gemm_mfma_rs: register-staged operands in the direct kernel's LDS formats
// ============================================================================
//
// For contiguous operands whose rows (LD_KU) or k-lines (LD_RU) are not
// 16-byte aligned, so the buffer unit cannot write them to LDS directly. Each
// thread fetches, with unaligned 16-byte global loads, the chunks that a
// direct load would have placed in its lane's LDS slots (the same KTile /
// RTile layouts and swizzles), and writes them there before the step's
// barrier; fragments, products and the pipeline are those of gemm_mfma_lds.
// Every load is branch-free: rows are clamped into the operand and, past K,
// k is clamped to the last chunk that lies inside it; the write to LDS undoes
// the clamp (the elements read early are shifted out, k past K becomes zeros;
// a k-contiguous operand's rows past the valid ones keep the clamped row,
// which only feeds accumulators outside C's view). The host sends a problem
// here only when the clamps stay inside the operand: K >= 8 for an LD_KU
// operand, and at least 8 rows (M or N) for an LD_RU operand.
template <int ROWS, int BK, int MODE, int NW, int R>
struct StagedLoader {
    static_assert(MODE == LD_KU || MODE == LD_RU, "contiguous operands");
    using KT = KTile<ROWS, BK>;
    using RT = RTile<ROWS, BK>;
    static constexpr int NLOADS = MODE == LD_KU ? KT::NLOADS : RT::NLOADS;
    static constexpr int PER = NLOADS / NW;
    static_assert(NLOADS % NW == 0, "wave loads must split evenly over the waves");

    u32x4 reg[R][PER];         // R register sets
    const uint16_t *origin;    // element (tile row 0, k = 0) of the operand
    int64_t srow, sk;          // element strides along rows and along k
    int kmax;                  // KU: K - 8 (last chunk start); RU: K - 1 (last k-line)
    int rows_valid;

    // The chunk (row, k) that wave load b puts in lane `lane`'s slot.
    __device__ static __forceinline__ void chunk(int b, int lane, int &row, int &k) {
        if constexpr (MODE == LD_KU) KT::src(b, lane, row, k);
        else RT::src(b, lane, k, row);
    }
    // LD_RU: rows the clamped load starts early (8 or more: none of its rows is valid).
    __device__ __forceinline__ int row_shift(int row) const { return min(row - min(row, rows_valid - 8), 8); }

    __device__ __forceinline__ void init(const uint16_t *origin_, int64_t srow_, int64_t sk_, int rows, int K) {
        origin = origin_;
        srow = srow_;
        sk = sk_;
        rows_valid = rows;
        kmax = MODE == LD_KU ? K - 8 : K - 1;
    }

    // Chunk addresses are recomputed per slice from the uniform origin and
    // strides (a few integer operations) rather than kept per chunk: the
    // 256x256 tile has no registers to spare.
    template <int SET>
    __device__ __forceinline__ void load(int k0, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            int row, kin;
            chunk(wave + NW * j, lane, row, kin);
            const int k = min(k0 + kin, kmax);
            if constexpr (MODE == LD_KU) {
                const int rc = row < rows_valid ? row : rows_valid - 1;
                reg[SET][j] = load16_unaligned(origin + (int64_t)rc * srow + k);
            } else {
                const int rc = min(row, rows_valid - 8);  // below the tile on one of fewer than 8 rows
                reg[SET][j] = load16_unaligned(origin + rc + (int64_t)k * sk);
            }
        }
    }

    // Writes set SET (the slice loaded for k0) into `tile` (this wave's
    // slots). CLAMP: some chunk may need its clamp undone (the slice reaches
    // past K, or the tile has fewer valid rows than ROWS); otherwise the
    // registers go to LDS as they are.
    template <int SET, bool CLAMP>
    __device__ __forceinline__ void store(char *tile, int k0, int wave, int lane) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            u32x4 v = reg[SET][j];
            if constexpr (CLAMP) {
                int row, kin;
                chunk(wave + NW * j, lane, row, kin);
                const int k = k0 + kin;
                if constexpr (MODE == LD_KU) {
                    // rows past the valid ones keep the clamped row's data:
                    // they only reach accumulators of C rows (or columns)
                    // outside the view, which are never stored
                    v = drop_elems(v, k - min(k, kmax));
                } else {
                    v = drop_elems(v, row_shift(row));
                    if (k > kmax) v = u32x4{0u, 0u, 0u, 0u};
                }
            }
            *reinterpret_cast<u32x4 *>(tile + (wave + NW * j) * 1024 + lane * 16) = v;
        }
    }

    __device__ __forceinline__ u32x4 frag(const char *tile, int r0, int k0, int lane) const {
        if constexpr (MODE == LD_KU) return frag_from_ktile<ROWS, BK>(tile, r0, k0, lane);
        else return frag_from_rtile<ROWS, BK>(tile, r0, k0, lane);
    }
};

// Register sets of the staged kernel: slice s is requested R steps before it
// is written to LDS (R steps of products cover its latency); S = R + 1 LDS
// stages. The 256x256x64 tile has room for one set only.
template <int BM, int BN, int BK>
constexpr int staged_sets() {
    return (BM * BN >= 256 * 256 && BK >= 64) ? 1 : (BM * BN >= 128 * 128 ? 2 : 3);
}

// WM x WN waves (every wave loads). One tile per workgroup only (no
// stream-K instantiation): written as a tile function called from the
// launch loop, the 256x256 tile's registers overflowed (the compiler spilled
// 4-31 registers, some inside the K loop), where this form spills none.
template <typename TI, int BM, int BN, int BK, int WM, int WN, int LA, int LB, int EM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mfma_rs(GemmArgs g) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int R = staged_sets<BM, BN, BK>();
    constexpr int S = R + 1;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 16 == 0, "tile shape");
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE];

    const WorkItem w = work_item(blockIdx.x, g);
    const int m0 = w.pm * BM, n0 = w.pn * BN;
    const int k_begin = w.split * g.k_chunk;
    const int kl = min(g.K - k_begin, g.k_chunk);  // this workgroup's K range
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    StagedLoader<BM, BK, LA, NW, R> la;
    StagedLoader<BN, BK, LB, NW, R> lb;
    const int rows_a = min(BM, g.M - m0), rows_b = min(BN, g.N - n0);
    la.init(static_cast<const uint16_t *>(g.A) + (int64_t)w.prod * g.bsa + (int64_t)m0 * g.sam +
                (int64_t)k_begin * g.sak,
            g.sam, g.sak, rows_a, kl);
    lb.init(static_cast<const uint16_t *>(g.B) + (int64_t)w.prod * g.bsb + (int64_t)n0 * g.sbn +
                (int64_t)k_begin * g.sbk,
            g.sbn, g.sbk, rows_b, kl);
    const bool edge = (LA == LD_RU && rows_a < BM) || (LB == LD_RU && rows_b < BN);  // an RU row clamp to undo

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (kl + BK - 1) / BK;
    constexpr int KSUB = BK / 16;
    u32x4 af[2][FM], bf[2][FN];
    auto fetch = [&](const char *stage, int kk, int set) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[set][j] = lb.frag(stage + A_BYTES, wn * WTN + j * 32, kk * 16, lane);
#pragma unroll
        for (int i = 0; i < FM; ++i) af[set][i] = la.frag(stage, wm * WTM + i * 32, kk * 16, lane);
    };
    auto mfmas = [&](int set, int from, int to) {
#pragma unroll
        for (int t = from; t < to; ++t) acc[t / FN][t % FN] = Mfma<TI>::run(af[set][t / FN], bf[set][t % FN], acc[t / FN][t % FN]);
    };
    // Writes slice k0 from register set SET into `stage`.
    auto commit = [&](auto set_tag, char *stage, int k0) {
        constexpr int SET = decltype(set_tag)::value;
        if (edge || k0 + BK > kl) {
            la.template store<SET, true>(stage, k0, wave, lane);
            sched_fence();  // one operand's shifts at a time (registers)
            lb.template store<SET, true>(stage + A_BYTES, k0, wave, lane);
        } else {
            la.template store<SET, false>(stage, k0, wave, lane);
            lb.template store<SET, false>(stage + A_BYTES, k0, wave, lane);
        }
    };
    auto load = [&](auto set_tag, int k0) {
        constexpr int SET = decltype(set_tag)::value;
        la.template load<SET>(k0, wave, lane);
        lb.template load<SET>(k0, wave, lane);
    };
    if (nk > 0) {
        // slices 0..R-1 into sets 0..R-1
        load(std::integral_constant<int, 0>{}, 0);
        if constexpr (R > 1) load(std::integral_constant<int, 1 % R>{}, BK);
        if constexpr (R > 2) load(std::integral_constant<int, 2 % R>{}, 2 * BK);
        commit(std::integral_constant<int, 0>{}, lds, 0);
        stage_barrier();
        fetch(lds, 0, 0);
    }
    constexpr int NMFMA = FM * FN;
    constexpr int NREAD = FM * (LA == LD_KU ? 1 : 2) + FN * (LB == LD_KU ? 1 : 2);
    constexpr int NLOAD = StagedLoader<BM, BK, LA, NW, R>::PER + StagedLoader<BN, BK, LB, NW, R>::PER;
    static_assert(KSUB % 2 == 0, "substep 0 of every slice uses fragment set 0");
    // Step kt over slice kt in stage `cur`: request slice kt+R into set kt%R
    // (a clamped dummy past K; the set's previous slice, kt, went to LDS in
    // the previous step), multiply, write slice kt+1 (set (kt+1)%R) into
    // stage `next` (last read R steps ago), synchronise, fetch the first
    // fragments of slice kt+1.
    auto step = [&](auto u_tag, char *__restrict__ cur, char *next, int kt) {
        constexpr int U = decltype(u_tag)::value;  // kt % R
        load(std::integral_constant<int, U>{}, (kt + R) * BK);
#pragma unroll
        for (int kk = 0; kk + 1 < KSUB; ++kk) {
            fetch(cur, kk + 1, (kk & 1) ^ 1);
            mfmas(kk & 1, 0, NMFMA);
        }
        constexpr int LAST = (KSUB - 1) & 1;
        mfmas(LAST, 0, NMFMA / 2);
        // the loads go out with the first substep's products
        interleave_mfma<NMFMA, NREAD, NLOAD>();
        interleave_mfma<NMFMA * (KSUB - 2), NREAD * (KSUB - 2), 0>();
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA / 2, 0);
        sched_fence();
        commit(std::integral_constant<int, (U + 1) % R>{}, next, (kt + 1) * BK);
        stage_barrier();
        sched_fence();
        fetch(next, 0, LAST ^ 1);
        mfmas(LAST, NMFMA / 2, NMFMA);
        interleave_mfma<NMFMA - NMFMA / 2, NREAD, 0>();
        sched_fence();
    };
    // R steps per iteration so the register set is a compile-time index; the
    // stages rotate at run time (slice kt lives in stage kt % S).
    static_assert(R >= 1 && R <= 3, "register sets");
    int kt = 0, cur = 0;
    auto step_u = [&](auto u_tag, int k) {
        const int nx = cur + 1 == S ? 0 : cur + 1;
        step(u_tag, lds + cur * STAGE, lds + nx * STAGE, k);
        cur = nx;
    };
    for (; kt + R <= nk; kt += R) {
        step_u(std::integral_constant<int, 0>{}, kt);
        if constexpr (R > 1) step_u(std::integral_constant<int, 1 % R>{}, kt + 1);
        if constexpr (R > 2) step_u(std::integral_constant<int, 2 % R>{}, kt + 2);
    }
    // fewer than R steps left; their register sets are 0, 1, ...
    if (kt < nk) step_u(std::integral_constant<int, 0>{}, kt);
    if constexpr (R > 2)
        if (kt + 1 < nk) step_u(std::integral_constant<int, 1 % R>{}, kt + 1);

    // The 256 x 256 register-staged kernels spill with GELU in the direct
    // epilogue (11 VGPRs), so theirs stays staged.
    finish_tile<EM, BM, BN, WM, WN, FM, FN, S * STAGE, (BM * BN < 256 * 256)>(g, w, acc, reinterpret_cast<float *>(lds),
                                                                          m0, n0);
}

// ============================================================================
// gemm_split_reduce: the second half of split-K
// ============================================================================
// One workgroup per (product, tile), the thread layout of the MFMA kernel that
// wrote the partials (WM x WN waves): thread t sums its float4s over the
// ranges in order 0..S-1 and holds the result in the accumulator layout, so
// the epilogue is the MFMA kernels' own write_tile. The loads of C ranges
// are issued together before any of their sums (a thread of a small tile
// holds only a few float4s, and one range at a time would cost one memory
// round trip per range); ranges past S-1 in the last group re-read range S-1
// and are not added.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_split_reduce(GemmArgs g) {
    constexpr int T = WM * WN * 64;
    constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
    constexpr int V = FM * FN * 4;
    constexpr int C = V >= 16 ? 1 : 16 / V;  // ranges in flight together
    constexpr int CAP = 64 * 1024;  // epilogue staging: at least 32 rows of every tile width
    __shared__ __attribute__((aligned(16))) float st[CAP / 4];

    const int tiles = g.grid_m * g.grid_n;
    WorkItem w;
    w.slot = blockIdx.x;
    w.prod = w.slot / tiles;
    w.split = 0;
    const int t = w.slot - w.prod * tiles;
    w.pm = t / g.grid_n;
    w.pn = t - w.pm * g.grid_n;
    const float4 *slot = reinterpret_cast<const float4 *>(g.ws) + (int64_t)w.slot * g.splits * (V * T);
    float4 sum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) sum[v] = slot[v * T + threadIdx.x];
    if constexpr (C == 1) {
        // Enough float4s per thread to keep the memory busy range by range.
#pragma unroll
        for (int v = 0; v < V; ++v)
            for (int s = 1; s < g.splits; ++s) {
                const float4 p = slot[((int64_t)s * V + v) * T + threadIdx.x];
                sum[v].x += p.x;
                sum[v].y += p.y;
                sum[v].z += p.z;
                sum[v].w += p.w;
            }
    } else {
        for (int s0 = 1; s0 < g.splits; s0 += C) {
            float4 p[C][V];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int s = min(s0 + c, g.splits - 1);
#pragma unroll
                for (int v = 0; v < V; ++v) p[c][v] = slot[((int64_t)s * V + v) * T + threadIdx.x];
            }
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (s0 + c < g.splits) {
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        sum[v].x += p[c][v].x;
                        sum[v].y += p[c][v].y;
                        sum[v].z += p[c][v].z;
                        sum[v].w += p[c][v].w;
                    }
                }
            }
        }
    }
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 t4 = sum[(i * FN + j) * 4 + q];
                acc[i][j][4 * q] = t4.x;
                acc[i][j][4 * q + 1] = t4.y;
                acc[i][j][4 * q + 2] = t4.z;
                acc[i][j][4 * q + 3] = t4.w;
            }
    write_tile<BM, BN, WM, WN, FM, FN, CAP>(g, w, acc, st, w.pm * BM, w.pn * BN);
}


// ============================================================================
// gemm_mfma_f32: fp32 inputs on the matrix cores (v_mfma_f32_32x32x2_f32)
// ============================================================================
// D[32x32] += A[32x2] * B[2x32]: lane l holds A[l % 32][l / 32] and
// B[l / 32][l % 32] (one fp32 each); the result layout is the 16-bit
// kernels'. A lane reads four consecutive k of its row from LDS (one
// ds_read_b128) and feeds them to four successive products: product j of an
// 8-k group takes k = 4 * (l / 32) + j, for A and B alike, so every k of the
// group is summed once (the k order within the 32 x 2 products only has to
// agree between the operands).
//
// Operands are staged through registers into LDS tiles [rows][BK + 4], k
// contiguous (the 4-float pad spreads the rows of a fragment read over the
// banks). The global loads per load mode:
//  LD_KC: k stride 1, rows 16-byte aligned, K % 4 == 0: 4-float chunks along
//         k, one 16-byte load each, written to LDS as they are;
//  LD_RC: row stride 1, k-lines 16-byte aligned, rows % 4 == 0: 4-float
//         chunks along the rows, one 16-byte load each, written to LDS as
//         four floats;
//  LD_GN: anything else, element loads through both strides.
// Every load is branch-free: its row and k are clamped into the operand (a
// chunk is wholly inside or wholly outside the view, given the mode's
// conditions), and store() writes zeros for what lies outside. A branch
// around a load would make the compiler wait for it where the paths join.
// Two register sets keep two slices in flight: slice kt+2 is requested at
// the top of step kt (slices past K re-read the last one) and written to LDS
// at the end of step kt+1.
template <int ROWS, int BK, int T, int MODE>
struct F32Loader {
    static_assert(MODE == LD_KC || MODE == LD_RC || MODE == LD_GN, "fp32 load modes");
    static constexpr int LDK = BK + 4;
    static constexpr int NCH = ROWS * BK / 4;  // 4-float chunks (KC, RC) per slice
    static constexpr int PER = MODE == LD_GN ? ROWS * BK / T : NCH / T;
    static_assert(MODE == LD_GN ? (ROWS * BK) % T == 0 : NCH % T == 0, "chunks split evenly over the threads");
    static constexpr int NREG = MODE == LD_GN ? PER : PER * 4;
    float reg[2][NREG];
    const float *base;  // element (row 0, k = 0) of the tile
    int64_t srow, sk;
    int rows_valid, K;  // >= 1 (>= 4 rows for LD_RC), >= 4 for LD_KC

    // The (row, k) of thread chunk c of a slice starting at k0.
    __device__ static __forceinline__ void chunk(int c, int tid, int k0, int &r, int &k) {
        const int q = c * T + tid;
        if constexpr (MODE == LD_KC) r = q / (BK / 4), k = k0 + (q % (BK / 4)) * 4;
        else if constexpr (MODE == LD_RC) k = k0 + q / (ROWS / 4), r = (q % (ROWS / 4)) * 4;
        else r = q / BK, k = k0 + q % BK;
    }

    template <int SET>
    __device__ __forceinline__ void load(int tid, int k0) {
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            int r, k;
            chunk(c, tid, k0, r, k);
            if constexpr (MODE == LD_KC) {
                const float4 v = *reinterpret_cast<const float4 *>(base + (int64_t)min(r, rows_valid - 1) * srow +
                                                                  min(k, K - 4));
                reg[SET][4 * c] = v.x, reg[SET][4 * c + 1] = v.y, reg[SET][4 * c + 2] = v.z, reg[SET][4 * c + 3] = v.w;
            } else if constexpr (MODE == LD_RC) {
                const float4 v = *reinterpret_cast<const float4 *>(base + (int64_t)min(k, K - 1) * sk +
                                                                  min(r, rows_valid - 4));
                reg[SET][4 * c] = v.x, reg[SET][4 * c + 1] = v.y, reg[SET][4 * c + 2] = v.z, reg[SET][4 * c + 3] = v.w;
            } else {
                reg[SET][c] = base[(int64_t)min(r, rows_valid - 1) * srow + (int64_t)min(k, K - 1) * sk];
            }
        }
    }

    template <int SET>
    __device__ __forceinline__ void store(int tid, int k0, float *lds) const {
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            int r, k;
            chunk(c, tid, k0, r, k);
            const bool in = r < rows_valid && k < K;
            if constexpr (MODE == LD_KC) {
                *reinterpret_cast<float4 *>(lds + r * LDK + (k - k0)) =
                    in ? make_float4(reg[SET][4 * c], reg[SET][4 * c + 1], reg[SET][4 * c + 2], reg[SET][4 * c + 3])
                       : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            } else if constexpr (MODE == LD_RC) {
#pragma unroll
                for (int e = 0; e < 4; ++e) lds[(r + e) * LDK + (k - k0)] = in ? reg[SET][4 * c + e] : 0.0f;
            } else {
                lds[r * LDK + (k - k0)] = in ? reg[SET][c] : 0.0f;
            }
        }
    }
};

template <int BM, int BN, int BK, int WM, int WN, int LA, int LB, int EM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mfma_f32(GemmArgs g) {
    constexpr int T = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LDK = BK + 4;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 8 == 0, "tile shape");
    constexpr int STAGE = (BM + BN) * LDK;  // floats
    __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

    const WorkItem w = work_item(blockIdx.x, g);
    const int m0 = w.pm * BM, n0 = w.pn * BN;
    const int k_begin = w.split * g.k_chunk;
    const int kl = min(g.K - k_begin, g.k_chunk);  // this workgroup's K range
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    F32Loader<BM, BK, T, LA> la;
    F32Loader<BN, BK, T, LB> lb;
    la.base = static_cast<const float *>(g.A) + (int64_t)w.prod * g.bsa + (int64_t)m0 * g.sam + (int64_t)k_begin * g.sak;
    la.srow = g.sam;
    la.sk = g.sak;
    la.rows_valid = min(BM, g.M - m0);
    la.K = kl;
    lb.base = static_cast<const float *>(g.B) + (int64_t)w.prod * g.bsb + (int64_t)n0 * g.sbn + (int64_t)k_begin * g.sbk;
    lb.srow = g.sbn;
    lb.sk = g.sbk;
    lb.rows_valid = min(BN, g.N - n0);
    lb.K = kl;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (kl + BK - 1) / BK;
    // This lane's fragment offsets (floats): row l % 32 of each 32-row block,
    // k = 4 * (l / 32) within each 8-k group.
    const int a_off = (wm * WTM + (lane & 31)) * LDK + 4 * (lane >> 5);
    const int b_off = BM * LDK + (wn * WTN + (lane & 31)) * LDK + 4 * (lane >> 5);
    auto multiply = [&](const float *s) {
#pragma unroll
        for (int kg = 0; kg < BK / 8; ++kg) {
            float4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const float4 *>(s + a_off + i * 32 * LDK + kg * 8);
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = *reinterpret_cast<const float4 *>(s + b_off + j * 32 * LDK + kg * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const float a = e == 0 ? af[i].x : e == 1 ? af[i].y : e == 2 ? af[i].z : af[i].w;
                        const float b = e == 0 ? bf[j].x : e == 1 ? bf[j].y : e == 2 ? bf[j].z : bf[j].w;
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i][j], 0, 0, 0);
                    }
        }
    };
    // Step kt (slice kt in LDS buffer kt & 1, set kt & 1 free): request slice
    // kt+2 into set kt & 1, multiply, write slice kt+1 (set (kt+1) & 1) into
    // the other buffer, synchronise. Two steps per iteration keep the set and
    // buffer indices compile-time.
    auto step = [&](auto u_tag, int kt) {
        constexpr int U = decltype(u_tag)::value;
        la.template load<U>(tid, (kt + 2) * BK);
        lb.template load<U>(tid, (kt + 2) * BK);
        multiply(lds + U * STAGE);
        if (kt + 1 < nk) {
            la.template store<U ^ 1>(tid, (kt + 1) * BK, lds + (U ^ 1) * STAGE);
            lb.template store<U ^ 1>(tid, (kt + 1) * BK, lds + (U ^ 1) * STAGE + BM * LDK);
        }
        __syncthreads();
    };
    if (nk > 0) {
        la.template load<0>(tid, 0);
        lb.template load<0>(tid, 0);
        la.template load<1>(tid, BK);
        lb.template load<1>(tid, BK);
        la.template store<0>(tid, 0, lds);
        lb.template store<0>(tid, 0, lds + BM * LDK);
        __syncthreads();
    }
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
    }
    if (kt < nk) step(std::integral_constant<int, 0>{}, kt);

    finish_tile<EM, BM, BN, WM, WN, FM, FN, (int)sizeof(lds)>(g, w, acc, lds, m0, n0);
}

}  // namespace dg
