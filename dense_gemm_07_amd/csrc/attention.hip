// Attention forward on gfx950 matrix cores: O = softmax(scale * Q K^T [causal]) V.
//
// The blockwise form of "如何用Triton手写Kernel优化矩阵乘与Flash Attention？"
// (the Flash Attention / online softmax section): one program per block of
// queries walks the keys in blocks, keeps a running maximum and a running sum
// of exponentials per query, rescales what it has accumulated when the
// maximum grows, and divides by the sum at the end, so the seq_q x seq_kv
// score matrix never leaves the chip.
//
// Mapping onto v_mfma_f32_32x32x16 (lane l, register r of a 32x32 result hold
// row 8*(r/4) + 4*(l/32) + r%4, column l%32):
//  - Each wave owns 32 queries. It computes S^T = K Q^T, so the 32 queries
//    are the result's columns: lane l always holds scores of query l%32. The
//    running max needs one exchange with lane l^32 per key block; the running
//    sum and the rescaling of O stay per lane.
//  - O^T += V^T P^T. The MFMA's k index only has to agree between its two
//    operands. K rows are loaded into LDS with bits 2 and 3 of the row
//    index swapped, which makes register r of S^T hold key 16*(r/8) +
//    8*(l/32) + r%8 of its 32-key block: registers 8t..8t+7 of a lane are
//    exactly the B operand (keys 8*(l/32) + e) of the t-th 16-key step. P
//    goes from the softmax straight into the second product, in registers.
//  - K (rows = keys, head_dim contiguous) and V (k = keys, rows = head_dim
//    contiguous) are moved global -> LDS by buffer loads into the GEMM's
//    swizzled tile formats, in a 3-stage ring: one barrier per key block.
//
// Numerics: fp32 scores and accumulators; exponentials through exp2 of the
// scores scaled by scale * log2(e); P is rounded to the input type for the
// second product (the matrix cores take 16-bit operands), the running sum
// adds the unrounded fp32 weights.
#include "attention.hpp"
#include "dg_kernels.hpp"

namespace dg {

// LDS row i of a K block holds key i with bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int attn_key_of_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <typename TI, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd(AttnArgs a) {
    constexpr int NW = 4;
    constexpr int BQ = kAttnBlockQ, BKV = kAttnBlockKV, S = kAttnStages;
    static_assert(BQ == NW * 32, "one 32-query column block per wave");
    using KT = KTile<BKV, D>;  // K block: rows = keys (permuted), k = head_dim
    using VT = RTile<D, BKV>;  // V block: k = keys, rows = head_dim
    constexpr int K_BYTES = BKV * D * 2, STAGE = 2 * BKV * D * 2;
    constexpr int K_PER = KT::NLOADS / NW, V_PER = VT::NLOADS / NW;
    static_assert(KT::NLOADS % NW == 0 && VT::NLOADS % NW == 0, "loads split evenly over the waves");
    constexpr int LOADS = K_PER + V_PER;  // per wave and key block
    constexpr int DK = D / 16;            // k-steps of K Q^T
    constexpr int DB = D / 32;            // 32-row blocks of O^T
    constexpr int SB = BKV / 32;          // 32-key blocks of S^T
    constexpr int PT = BKV / 16;          // k-steps of V^T P^T
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE];

    const int bh_count = a.batch * a.heads;
    const int qi = blockIdx.x / bh_count, bh = blockIdx.x - qi * bh_count;
    const int qblk = CAUSAL ? a.q_blocks - 1 - qi : qi;  // causal: the longest rows start first
    const int b = bh / a.heads, h = bh - b * a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int q0 = qblk * BQ;
    const int wq0 = q0 + wave * 32;      // this wave's first query
    const int my_q = wq0 + (lane & 31);  // this lane's query

    const uint16_t *Qp = static_cast<const uint16_t *>(a.Q) + (int64_t)b * a.qb + (int64_t)h * a.qh;
    const uint16_t *Kp = static_cast<const uint16_t *>(a.K) + (int64_t)b * a.kb + (int64_t)h * a.kh;
    const uint16_t *Vp = static_cast<const uint16_t *>(a.V) + (int64_t)b * a.vb + (int64_t)h * a.vh;

    // Q^T as the B operand of S^T = K Q^T: lane l holds Q[my_q][16kk + 8*(l/32) + e].
    u32x4 qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qf[kk] = my_q < a.seq_q ? *reinterpret_cast<const u32x4 *>(Qp + (int64_t)my_q * a.qs + 16 * kk + 8 * half)
                                : u32x4{0u, 0u, 0u, 0u};

    // Buffer-load descriptors and this lane's share of each block's loads.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)Kp, 0, kNumRecords, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)Vp, 0, kNumRecords, kRsrcWord3);
    int kkey[K_PER], kvo[K_PER], vkey[V_PER], vvo[V_PER];
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
        int row, k;
        KT::src(wave + NW * j, lane, row, k);
        kkey[j] = attn_key_of_row(row);
        kvo[j] = (int)(2 * ((int64_t)kkey[j] * a.ks + k));
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
        int k, row;
        VT::src(wave + NW * j, lane, k, row);
        vkey[j] = k;
        vvo[j] = (int)(2 * ((int64_t)k * a.vs + row));
    }
    // Queue key block [kv0, kv0 + BKV) into `stage`; keys past seq_kv load zeros.
    auto issue = [&](char *stage, int kv0) {
#pragma unroll
        for (int j = 0; j < K_PER; ++j) {
            const int vo = kv0 + kkey[j] < a.seq_kv ? kvo[j] : kOobOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_t *)(stage + (wave + NW * j) * 1024), 16, vo,
                                                     (int)(2 * (int64_t)kv0 * a.ks), 0, 0);
        }
#pragma unroll
        for (int j = 0; j < V_PER; ++j) {
            const int vo = kv0 + vkey[j] < a.seq_kv ? vvo[j] : kOobOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_t *)(stage + K_BYTES + (wave + NW * j) * 1024),
                                                     16, vo, (int)(2 * (int64_t)kv0 * a.vs), 0, 0);
        }
    };

    int nkv = (a.seq_kv + BKV - 1) / BKV;
    if (CAUSAL) nkv = min(nkv, (min(a.seq_q, q0 + BQ) - 1) / BKV + 1);  // keys beyond the block's last query

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -__builtin_inff();  // running max of the log2-scaled scores of my_q
    float l = 0.0f;               // running sum of this lane's weights (its half of the keys)

    // One key block: scores, online softmax update, O^T += V^T P^T. The stage
    // pointers never alias the stage being filled (restrict keeps the
    // compiler from waiting on those loads before reading these).
    auto block = [&](const char *__restrict__ kt, const char *__restrict__ vt, int kv0) {
        f32x16 s[SB];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[sb][r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk)
                s[sb] = Mfma<TI>::run(frag_from_ktile<BKV, D>(kt, 32 * sb, 16 * kk, lane), qf[kk], s[sb]);
        }
        float mb = -__builtin_inff();
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * sb + 16 * (r >> 3) + 8 * half + (r & 7);
                float t = s[sb][r] * a.scale_log2;
                if (key >= a.seq_kv || (CAUSAL && key > my_q)) t = -__builtin_inff();
                s[sb][r] = t;
                mb = fmaxf(mb, t);
            }
        mb = fmaxf(mb, __shfl_xor(mb, 32));
        const float mn = fmaxf(m, mb);
        const float mu = mn == -__builtin_inff() ? 0.0f : mn;  // nothing allowed yet: weights stay 0
        const float alpha = __builtin_amdgcn_exp2f(m - mu);
        float ps = 0.0f;
        u32x4 pf[PT];
#pragma unroll
        for (int t = 0; t < PT; ++t) {
            uint16_t e8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(s[t >> 1][8 * (t & 1) + e] - mu);
                ps += p;
                e8[e] = from_f32<TI>(p);
            }
            pf[t] = pack8(e8);
        }
        l = l * alpha + ps;
        m = mn;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
        for (int t = 0; t < PT; ++t)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = Mfma<TI>::run(frag_from_rtile<D, BKV>(vt, 32 * db, 16 * t, lane), pf[t], o[db]);
    };

#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(lds + s * STAGE, s * BKV);
    int cur = 0;
    for (int kb = 0; kb < nkv; ++kb) {
        wait_vmcnt<(S - 2) * LOADS>();  // block kb has landed (this wave's loads)
        stage_barrier();                // ... everyone's; and everyone is done with block kb-1
        const int fill = cur == 0 ? S - 1 : cur - 1;
        issue(lds + fill * STAGE, (kb + S - 1) * BKV);
        const int kv0 = kb * BKV;
        // causal: a wave whose queries all precede the block has nothing to add
        if (!CAUSAL || kv0 <= wq0 + 31) block(lds + cur * STAGE, lds + cur * STAGE + K_BYTES, kv0);
        cur = cur + 1 == S ? 0 : cur + 1;
    }
    wait_vmcnt<0>();  // the trailing out-of-range loads land before the workgroup exits

    // O = O^T / l (lane l holds query my_q, head_dim rows 32db + 8*(r/4) + 4*(l/32) + r%4)
    const float lt = l + __shfl_xor(l, 32);
    if (my_q >= a.seq_q) return;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    char *Op = static_cast<char *>(a.O);
    const int es = a.out_dtype == DG_F32 ? 4 : 2;
    const int64_t orow = ((int64_t)b * a.ob + (int64_t)h * a.oh + (int64_t)my_q * a.os) * es;
    const bool vec = (((uintptr_t)Op + orow) % (uintptr_t)(4 * es)) == 0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * db + 8 * r4 + 4 * half;
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = o[db][4 * r4 + e] * inv;
            char *p = Op + orow + (int64_t)d0 * es;
            if (a.out_dtype == DG_F32) store4_t<DG_F32>(p, vec, 4, 1, y);
            else if (a.out_dtype == DG_BF16) store4_t<DG_BF16>(p, vec, 4, 1, y);
            else store4_t<DG_F16>(p, vec, 4, 1, y);
        }
    if (a.lse && half == 0)
        a.lse[((int64_t)b * a.heads + h) * a.seq_q + my_q] =
            lt > 0.0f ? (m + __log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
}

template <typename TI, int D, bool CAUSAL>
static void launch_t(const AttnArgs &a, hipStream_t s) {
    const unsigned groups = (unsigned)a.batch * (unsigned)a.heads * (unsigned)a.q_blocks;
    hipLaunchKernelGGL((attn_fwd<TI, D, CAUSAL>), dim3(groups), dim3(256), 0, s, a);
}

hipError_t launch_attention(const AttnArgs &a, int in_dtype, int head_dim, hipStream_t s) {
    if (head_dim != 64) return hipErrorInvalidValue;
    if (in_dtype == DG_BF16) {
        if (a.causal) launch_t<BF16, 64, true>(a, s);
        else launch_t<BF16, 64, false>(a, s);
    } else if (in_dtype == DG_F16) {
        if (a.causal) launch_t<F16, 64, true>(a, s);
        else launch_t<F16, 64, false>(a, s);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dg
