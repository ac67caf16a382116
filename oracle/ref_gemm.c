/*
 * Plain fp64 CPU oracle for the dense matrix product C = A @ B, its fused
 * epilogue, and the attention forward pass (softmax(Q K^T) V).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or helper with
 * the HIP library; it is built by gcc on its own.
 *
 * What it computes (the plain definition, not a tiled emulation):
 *   C[i][j] = sum_{k=0..K-1} A[i][k] * B[k][j]
 * -- "I Wrote a GPU Matmul Kernel From Scratch in Triton", Step 1 (the
 *    three-loop naive matmul, C zero-initialised, M*N*K multiplies), and
 *    "用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到 MatMul" §3.1 (one
 *    output element is a row of A times a column of B, summed over K).
 * Tiling, splitting K into BLOCK_K slices and reordering the output tiles are
 * exact regroupings of this sum (same pages, Step 2 and §3.3 "C_tile =
 * A0B0 + A1B1"), so the oracle is the definition itself.
 *
 * Readings taken where the pages leave a step open:
 *  - Inputs are fp32, fp16 or bf16 values. They are decoded to fp64 exactly,
 *    from the IEEE-754 bit layouts, and every product of two such values is
 *    exact in fp64; only the additions round. Sum order is k ascending,
 *    starting from +0.0.
 *  - Element addressing goes through element strides: A[i][k] sits at
 *    i*sam + k*sak, B[k][j] at k*sbk + j*sbn ("Triton：04 Matmul、Autotune 与
 *    PyTorch 集成", the teaching kernel's stride arguments; "用 Triton 写 GPU
 *    Kernel" §4.1, offsets count elements, not bytes).
 *  - Elements outside the M x N x K view are never read (masked loads fill
 *    zero, which adds nothing: "用 Triton 写 GPU Kernel" §4.6).
 *  - K = 0 gives the empty sum +0.0.
 *  - Output rounding to fp16/bf16/fp32 is round-to-nearest-even, written out
 *    here from the bit layouts (the pages cast the fp32 accumulator with
 *    acc.to(tl.float16), §4.5/§4.6 of the same page; the rounding rule is the
 *    IEEE default).
 *
 * Threads: rows of C are shared out over OpenMP threads; that changes no
 * arithmetic (each C[i][j] is one sequential sum).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Oracle-local dtype codes (the caller passes these; they are this file's own). */
enum { REF_F32 = 0, REF_F16 = 1, REF_BF16 = 2 };

/* ---- decoding: bit pattern -> exact fp64 value ---------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)            v = ldexp((double)f, -24);            /* zero / subnormal */
    else if (e == 0x1f)    v = f ? NAN : INFINITY;
    else                   v = ldexp((double)(1024 + f), e - 25); /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double dec_bf16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)            v = ldexp((double)f, -133);           /* zero / subnormal */
    else if (e == 0xff)    v = f ? NAN : INFINITY;
    else                   v = ldexp((double)(128 + f), e - 134); /* 1.f * 2^(e-127) */
    return sign ? -v : v;
}

/* binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits. */
static double dec_f32(uint32_t w) {
    int sign = (w >> 31) & 1;
    int e = (w >> 23) & 0xff;
    uint32_t f = w & 0x7fffff;
    double v;
    if (e == 0)            v = ldexp((double)f, -149);
    else if (e == 0xff)    v = f ? NAN : INFINITY;
    else                   v = ldexp((double)(0x800000u + f), e - 150);
    return sign ? -v : v;
}

static double dec_at(int dtype, const void *base, int64_t idx) {
    switch (dtype) {
    case REF_F16:  return dec_f16(((const uint16_t *)base)[idx]);
    case REF_BF16: return dec_bf16(((const uint16_t *)base)[idx]);
    default:       return dec_f32(((const uint32_t *)base)[idx]);
    }
}

/* ---- encoding: fp64 value -> nearest representable, ties to even --------- */

/* Round a non-negative finite x to a format with `p` significand bits,
 * minimum normal exponent emin and maximum exponent emax, returning the
 * biased-exponent/fraction bit field (without sign), or the infinity field
 * on overflow. `bias` is the exponent bias, `fbits` = p - 1. */
static uint32_t enc_mag(double x, int p, int emin, int emax, int bias) {
    int fbits = p - 1;
    uint32_t inf_field = (uint32_t)((2 * bias + 1)) << fbits;
    if (x == 0.0) return 0;
    int E;
    frexp(x, &E);            /* x = m * 2^E, m in [0.5, 1): x's exponent is E-1 */
    int e = E - 1;
    if (e < emin) e = emin;  /* subnormal range: fixed quantum 2^(emin - fbits) */
    /* scaled significand: x / 2^(e - fbits), exact (power-of-two scaling) */
    double s = ldexp(x, fbits - e);
    double q = nearbyint(s); /* default rounding mode: to nearest, ties to even */
    if (q >= ldexp(1.0, p)) { /* rounded up to the next binade */
        q = ldexp(1.0, fbits);
        e += 1;
    }
    if (q < ldexp(1.0, fbits)) {
        /* subnormal (e == emin and no implicit bit) */
        return (uint32_t)q;
    }
    if (e > emax) return inf_field;
    uint32_t biased = (uint32_t)(e + bias);
    return (biased << fbits) | ((uint32_t)q - (1u << fbits));
}

static uint16_t enc_f16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7e00;
    if (isinf(x)) return sign | 0x7c00;
    return sign | (uint16_t)enc_mag(fabs(x), 11, -14, 15, 15);
}

static uint16_t enc_bf16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7fc0;
    if (isinf(x)) return sign | 0x7f80;
    return sign | (uint16_t)enc_mag(fabs(x), 8, -126, 127, 127);
}

static uint32_t enc_f32(double x) {
    uint32_t sign = signbit(x) ? 0x80000000u : 0;
    if (isnan(x)) return sign | 0x7fc00000u;
    if (isinf(x)) return sign | 0x7f800000u;
    return sign | enc_mag(fabs(x), 24, -126, 127, 127);
}

/* ---- exported entry points (ctypes) --------------------------------------- */

int ref_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Decode n contiguous elements of `dtype` into fp64. */
void ref_decode(int dtype, const void *src, int64_t n, double *dst) {
    for (int64_t t = 0; t < n; ++t) dst[t] = dec_at(dtype, src, t);
}

/* Round n fp64 values to `dtype` (nearest, ties to even); write bit patterns. */
void ref_encode(int dtype, const double *src, int64_t n, void *dst) {
    for (int64_t t = 0; t < n; ++t) {
        if (dtype == REF_F16)       ((uint16_t *)dst)[t] = enc_f16(src[t]);
        else if (dtype == REF_BF16) ((uint16_t *)dst)[t] = enc_bf16(src[t]);
        else                        ((uint32_t *)dst)[t] = enc_f32(src[t]);
    }
}

/*
 * Full product. A and B are read through element strides; C is written as a
 * row-major M x N fp64 array with leading dimension ldc.
 * The operands are first decoded into fp64 copies (A as rows of K values, B
 * as columns of K values, so each dot product walks two contiguous arrays);
 * the decode is exact, so this is a change of storage, not of arithmetic.
 * Returns 0, or -1 if the copies cannot be allocated.
 */
int ref_gemm(int64_t M, int64_t N, int64_t K, int dtype,
             const void *A, int64_t sam, int64_t sak,
             const void *B, int64_t sbk, int64_t sbn,
             double *C, int64_t ldc) {
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *bt = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!a || !bt) { free(a); free(bt); return -1; }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) a[i * K + k] = dec_at(dtype, A, i * sam + k * sak);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) bt[j * K + k] = dec_at(dtype, B, k * sbk + j * sbn);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        const double *ai = a + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const double *bj = bt + j * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += ai[k] * bj[k];
            C[i * ldc + j] = s;
        }
    }
    free(a);
    free(bt);
    return 0;
}

/*
 * Selected entries only: out[t] = C[rows[t]][cols[t]], each computed straight
 * from the definition (decode on the fly, k ascending). For sampling outputs
 * of problems too large for the full product.
 */
void ref_gemm_entries(int64_t K, int dtype,
                      const void *A, int64_t sam, int64_t sak,
                      const void *B, int64_t sbk, int64_t sbn,
                      int64_t n, const int64_t *rows, const int64_t *cols,
                      double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += dec_at(dtype, A, i * sam + k * sak) * dec_at(dtype, B, k * sbk + j * sbn);
        out[t] = s;
    }
}

/*
 * Whole rows [row0, row0 + nrows) of C, each entry straight from the
 * definition, written row-major with leading dimension N. Used to time the
 * oracle on a bounded slice of a large problem.
 */
void ref_gemm_rows(int64_t row0, int64_t nrows, int64_t N, int64_t K, int dtype,
                   const void *A, int64_t sam, int64_t sak,
                   const void *B, int64_t sbk, int64_t sbn,
                   double *out) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t j = 0; j < N; ++j) {
            int64_t i = row0 + r;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += dec_at(dtype, A, i * sam + k * sak) * dec_at(dtype, B, k * sbk + j * sbn);
            out[r * N + j] = s;
        }
}

/*
 * Fused epilogue over a product P already computed above (row-major fp64,
 * leading dimension ldp):
 *
 *   out[i][j] = act(alpha * P[i][j] + beta * R[i][j] + bias)
 *
 * The pages name the two uses this serves -- the product standing in for a
 * linear layer ("如何用Triton手写Kernel优化矩阵乘与Flash Attention？",
 * 性能对比与工程落地建议) and element-wise steps fused into the kernel that
 * produces their input ("用 Triton 写 GPU Kernel：从 Vector Add、Softmax 到
 * MatMul", §2.7) -- but give no formula. Reading taken: the BLAS form
 * alpha*P + beta*R, plus a bias broadcast along rows (bias[j], per column) or
 * along columns (bias[i], per row), then an activation, all in fp64 in the
 * order written, rounded once by the caller.
 *  - alpha and beta are the fp32 values the caller passes (exact in fp64).
 *  - beta == 0: R is not read (a NaN in R does not reach the result).
 *  - R[i][j] at R + i*srm + j*srn, bias at bias + (per_row ? i : j)*sbias,
 *    decoded exactly like A and B. bias == NULL: no bias.
 *  - act 0: none. act 1: ReLU, v < 0 -> +0, anything else (NaN, -0) kept.
 *    act 2: GELU, v * Phi(v) with Phi the standard normal CDF,
 *    Phi(v) = erfc(-v / sqrt(2)) / 2 (C99 erfc in fp64).
 */
static double ref_act(double v, int act) {
    if (act == 1) return v < 0.0 ? 0.0 : v;
    if (act == 2) return v * 0.5 * erfc(-v / sqrt(2.0));
    return v;
}

void ref_epilogue(int64_t M, int64_t N, const double *P, int64_t ldp,
                  double alpha, double beta,
                  int r_dtype, const void *R, int64_t srm, int64_t srn,
                  int bias_dtype, const void *bias, int64_t sbias, int per_row,
                  int act, double *out, int64_t ldo) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * P[i * ldp + j];
            if (beta != 0.0) v += beta * dec_at(r_dtype, R, i * srm + j * srn);
            if (bias) v += dec_at(bias_dtype, bias, (per_row ? i : j) * sbias);
            out[i * ldo + j] = ref_act(v, act);
        }
}

/*
 * Attention forward, the plain definition, for every (batch b, head h):
 *
 *   s[i][j] = scale * sum_d Q[i][d] K[j][d]            for allowed j
 *   O[i][:] = sum_j exp(s[i][j] - m_i) V[j][:] / l_i,   m_i = max_j s[i][j],
 *             l_i = sum_j exp(s[i][j] - m_i),           lse_i = m_i + log(l_i)
 *
 * ("如何用Triton手写Kernel优化矩阵乘与Flash Attention？", the section on Flash
 * Attention and online softmax: scores are a block of Q times K transposed
 * divided by sqrt(head_dim), softmax along the keys, then a weighted sum of
 * V; the blockwise running-max form computes the same softmax.) Readings:
 *  - allowed j: all j < seq_kv; with causal != 0 only j <= i (the page's
 *    causal mask keeps keys whose index does not exceed the query's;
 *    excluded keys get weight exactly 0);
 *  - softmax subtracts the row maximum first (the stable form), in fp64;
 *  - Q, K, V elements at ptr + b*sb + h*sh + row*ss + d (element strides,
 *    d stride 1), decoded exactly; O and lse are row-major fp64
 *    [batch][heads][seq_q][head_dim] and [batch][heads][seq_q].
 */
int ref_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_kv, int64_t dim, int dtype,
                  const void *Q, int64_t qb, int64_t qh, int64_t qs,
                  const void *K, int64_t kb, int64_t kh, int64_t ks,
                  const void *V, int64_t vb, int64_t vh, int64_t vs,
                  double scale, int causal, double *O, double *lse) {
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(seq_kv > 0 ? seq_kv : 1));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t h = 0; h < heads; ++h)
                for (int64_t i = 0; i < seq_q; ++i) {
                    if (!s) continue;
                    const int64_t qo = b * qb + h * qh + i * qs;
                    const int64_t n = causal ? (i + 1 < seq_kv ? i + 1 : seq_kv) : seq_kv;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < n; ++j) {
                        const int64_t ko = b * kb + h * kh + j * ks;
                        double dot = 0.0;
                        for (int64_t d = 0; d < dim; ++d) dot += dec_at(dtype, Q, qo + d) * dec_at(dtype, K, ko + d);
                        s[j] = scale * dot;
                        if (s[j] > m) m = s[j];
                    }
                    double l = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        s[j] = exp(s[j] - m);
                        l += s[j];
                    }
                    double *o = O + ((b * heads + h) * seq_q + i) * dim;
                    for (int64_t d = 0; d < dim; ++d) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < n; ++j) acc += s[j] * dec_at(dtype, V, b * vb + h * vh + j * vs + d);
                        o[d] = n > 0 ? acc / l : 0.0;
                    }
                    if (lse) lse[(b * heads + h) * seq_q + i] = n > 0 ? m + log(l) : -INFINITY;
                }
        free(s);
    }
    return fail ? -1 : 0;
}
