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
//  - Each wave owns kAttnQueryGroups groups of 32 queries. It computes
//    S^T = K Q^T, so a group's 32 queries are the result's columns: lane l
//    always holds scores of query l%32 of each group. The running max needs
//    one exchange with lane l^32 per key block; the running sum and the
//    rescaling of O stay per lane. Each K or V fragment read from LDS feeds
//    every group's MFMA.
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
// adds the unrounded fp32 weights. The maximum subtracted in the exponent is
// a reference that moves only when a block's weights against it would grow
// large (their sum past 2^8): the page's rescaling runs then, not on every
// growth of the maximum, which gives the same result up to rounding.
#include <type_traits>

#include "attention.hpp"
#include "dg_kernels.hpp"

namespace dg {

// LDS row i of a K block holds key i with bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int attn_key_of_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// c * max(x of lane l, x of lane l ^ 32) in every lane, for c > 0: gfx950
// swaps the upper half of one register with the lower half of another in one
// VALU instruction, which spares a round trip through LDS. Scaling each half
// first gives the same value (rounding is monotone) and spares the moves that
// fmaxf needs on values of unknown origin.
__device__ __forceinline__ float scaled_max_of_halves(float x, float c) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]) * c, __uint_as_float(r[1]) * c);
}

// One lane's weights of a key block, exp2(c * s + nm) for its 16 * SB
// scores, rounded to the input type and packed as the B operands of the
// product with V (register 8t + e of the scores is key e of 16-key step t),
// and their sum in fp32. The scale folds into the exponent's fused
// multiply-add.
template <typename TI, int SB>
__device__ __forceinline__ float attn_weights(const f32x16 (&s)[SB], u32x4 (&pf)[2 * SB], float c, float nm) {
    float ps = -0.0f;  // -0 + p is p: the first addition folds away
#pragma unroll
    for (int t = 0; t < 2 * SB; ++t) {
        uint16_t e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t >> 1][8 * (t & 1) + e], c, nm));
            ps += p;
            e8[e] = from_f32<TI>(p);
        }
        pf[t] = pack8(e8);
    }
    return ps;
}

template <typename TI, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd(AttnArgs a) {
    constexpr int NW = 4;
    constexpr int QG = kAttnQueryGroups;  // 32-query groups per wave
    constexpr int BQ = kAttnBlockQ, BKV = kAttnBlockKV, S = attn_stages(D);
    static_assert(BQ == NW * 32 * QG, "QG 32-query column blocks per wave");
    static_assert(D % 64 == 0, "head_dim in whole 64-column K tiles");
    // K block: rows = keys (permuted), k = head_dim, stored as D/64 tiles of
    // 64 columns (the tile format's rows are 128 bytes). V block: k = keys,
    // rows = head_dim.
    constexpr int KH = D / 64;
    using KT = KTile<BKV, 64>;
    using VT = RTile<D, BKV>;
    constexpr int K_HALF = BKV * 64 * 2;  // bytes of one 64-column K tile
    constexpr int K_BYTES = KH * K_HALF, STAGE = 2 * BKV * D * 2;
    constexpr int K_PER = KH * KT::NLOADS / NW, V_PER = VT::NLOADS / NW;
    static_assert((KH * KT::NLOADS) % NW == 0 && VT::NLOADS % NW == 0, "loads split evenly over the waves");
    constexpr int LOADS = K_PER + V_PER;  // per wave and key block
    constexpr int DK = D / 16;            // k-steps of K Q^T
    constexpr int DB = D / 32;            // 32-row blocks of O^T
    constexpr int SB = BKV / 32;          // 32-key blocks of S^T
    constexpr int PT = BKV / 16;          // k-steps of V^T P^T
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE];

    // Workgroup order. Without a mask: the ids one XCD receives (they are
    // dealt round-robin) get consecutive logical numbers, and consecutive
    // numbers walk the query blocks of one (batch, head). An XCD then works
    // on one or two heads at a time, whose workgroups read the same K/V
    // blocks at about the same time, so its L2 serves most of them: a tenth
    // of the fabric traffic of the head-fastest order, which put eight heads
    // on each XCD at once (16 MiB of K/V against a 4 MiB L2 at seq 8192).
    // Causal: the same XCD numbering, then groups of four heads whose query
    // blocks run longest first, the group's heads interleaved, so that short
    // blocks fill in behind long ones (walking one head at a time left each
    // XCD's last long blocks to start late: 6 % slower; all heads at once,
    // longest first, read twice the K/V bytes from beyond the L2).
    int bh, qi;
    const int lid = a.num_xcd > 1 ? xcd_rank(blockIdx.x, gridDim.x, a.num_xcd) : blockIdx.x;
    if (CAUSAL) {
        // Groups of G heads, each group's query blocks longest first with
        // its heads interleaved: the XCD's working set is G heads' K/V, and
        // the next group's long blocks start while this group's short ones
        // still run.
        constexpr int G = 4;
        const int bh_count = a.batch * a.heads;
        const int group = lid / (G * a.q_blocks);
        const int gh = min(G, bh_count - group * G);  // heads in this group
        const int r = lid - group * G * a.q_blocks;
        qi = r / gh;
        bh = group * G + (r - qi * gh);
    } else {
        bh = lid / a.q_blocks;
        qi = lid - bh * a.q_blocks;
    }
    const int qblk = CAUSAL ? a.q_blocks - 1 - qi : qi;  // causal: the longest rows start first
    const int b = bh / a.heads, h = bh - b * a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int q0 = qblk * BQ;
    const int wq0 = q0 + wave * 32 * QG;  // this wave's first query; group g holds wq0 + 32g + (l % 32)
    int my_q[QG];
#pragma unroll
    for (int g = 0; g < QG; ++g) my_q[g] = wq0 + 32 * g + (lane & 31);

    const uint16_t *Qp = static_cast<const uint16_t *>(a.Q) + (int64_t)b * a.qb + (int64_t)h * a.qh;
    const uint16_t *Kp = static_cast<const uint16_t *>(a.K) + (int64_t)b * a.kb + (int64_t)h * a.kh;
    const uint16_t *Vp = static_cast<const uint16_t *>(a.V) + (int64_t)b * a.vb + (int64_t)h * a.vh;

    // Q^T as the B operand of S^T = K Q^T: lane l holds Q[query][16kk + 8*(l/32) + e].
    u32x4 qf[QG][DK];
#pragma unroll
    for (int g = 0; g < QG; ++g)
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            qf[g][kk] = my_q[g] < a.seq_q
                            ? *reinterpret_cast<const u32x4 *>(Qp + (int64_t)my_q[g] * a.qs + 16 * kk + 8 * half)
                            : u32x4{0u, 0u, 0u, 0u};

    // Buffer-load descriptors and this lane's share of each block's loads.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)Kp, 0, kNumRecords, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)Vp, 0, kNumRecords, kRsrcWord3);
    int kkey[K_PER], kvo[K_PER], vkey[V_PER], vvo[V_PER];
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
        const int bl = wave + NW * j;  // wave load bl fills 1 KiB at byte bl * 1024: tile bl / NLOADS
        int row, k;
        KT::src(bl % KT::NLOADS, lane, row, k);
        kkey[j] = attn_key_of_row(row);
        kvo[j] = (int)(2 * ((int64_t)kkey[j] * a.ks + 64 * (bl / KT::NLOADS) + k));
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
        int k, row;
        VT::src(wave + NW * j, lane, k, row);
        vkey[j] = k;
        vvo[j] = (int)(2 * ((int64_t)k * a.vs + row));
    }
    // Every helper lambda below is forced inline: left to the inliner, the
    // unrolled key loop's block became a call, and the kernel's arguments
    // went through scratch memory.
    //
    // Queue key block [kv0, kv0 + BKV) into `stage`; with CHECK, keys past
    // seq_kv load zeros (without, the caller knows the block lies inside).
    auto issue = [&](auto check_tag, char *stage, int kv0) __attribute__((always_inline)) {
        constexpr bool CHECK = decltype(check_tag)::value;
#pragma unroll
        for (int j = 0; j < K_PER; ++j) {
            const int vo = !CHECK || kv0 + kkey[j] < a.seq_kv ? kvo[j] : kOobOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_t *)(stage + (wave + NW * j) * 1024), 16, vo,
                                                     (int)(2 * (int64_t)kv0 * a.ks), 0, 0);
        }
#pragma unroll
        for (int j = 0; j < V_PER; ++j) {
            const int vo = !CHECK || kv0 + vkey[j] < a.seq_kv ? vvo[j] : kOobOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_t *)(stage + K_BYTES + (wave + NW * j) * 1024),
                                                     16, vo, (int)(2 * (int64_t)kv0 * a.vs), 0, 0);
        }
    };

    int nkv = (a.seq_kv + BKV - 1) / BKV;
    if (CAUSAL) nkv = min(nkv, (min(a.seq_q, q0 + BQ) - 1) / BKV + 1);  // keys beyond the block's last query

    f32x16 o[QG][DB];
#pragma unroll
    for (int g = 0; g < QG; ++g)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[g][db][r] = 0.0f;
    // m: the reference max of the log2-scaled scores (-inf until a key is
    // allowed); nmu: -m, or +inf while m is -inf (which makes the next
    // block's weights overflow and so move m); l: this lane's running sum
    // (its half of the keys).
    float m[QG], nmu[QG], l[QG];
#pragma unroll
    for (int g = 0; g < QG; ++g) m[g] = -__builtin_inff(), nmu[g] = __builtin_inff(), l[g] = 0.0f;

    // Scores of one key block: S^T = K Q^T for the wave's query groups.
    auto qk = [&](const char *__restrict__ kt, f32x16 (&s)[QG][SB]) __attribute__((always_inline)) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
            for (int g = 0; g < QG; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[g][sb][r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const u32x4 kf = frag_from_ktile<BKV, 64>(kt + (kk / 4) * K_HALF, 32 * sb, 16 * (kk % 4), lane);
#pragma unroll
                for (int g = 0; g < QG; ++g) s[g][sb] = Mfma<TI>::run(kf, qf[g][kk], s[g][sb]);
            }
        }
    };

    // Online softmax update of one key block's scores, then O^T += V^T P^T.
    // MASK: the block holds keys past seq_kv or past some query of the wave
    // (causal); interior blocks skip the per-score test.
    auto softmax_pv = [&](auto mask_tag, f32x16 (&s)[QG][SB], const char *__restrict__ vt,
                          int kv0) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        u32x4 pf[QG][PT];
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            if constexpr (MASK) {
#pragma unroll
                for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * sb + 16 * (r >> 3) + 8 * half + (r & 7);
                        if (key >= a.seq_kv || (CAUSAL && key > my_q[g])) s[g][sb][r] = -__builtin_inff();
                    }
            }
            // Weights against the reference max m held so far. O, l and lse
            // are all relative to m, so any m gives the same result up to
            // rounding, as long as no weight overflows: their sum (every
            // weight is >= 0) bounds each of them. Only when some lane's sum
            // exceeds 2^8 (a wave vote; also on a query's first allowed
            // keys, where nmu is +inf and the sum inf or NaN) does the block
            // max move m, rescale O and l, and the weights get recomputed.
            // With random scores that happens in the first blocks only.
            float ps = attn_weights<TI>(s[g], pf[g], a.scale_log2, nmu[g]);
            if (__any(!(ps <= kAttnSumLimit))) {
                // The max is taken on the raw scores (scale > 0 keeps their order).
                float mb = -__builtin_inff();
#pragma unroll
                for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s[g][sb][r]);
                mb = scaled_max_of_halves(mb, a.scale_log2);
                const float mn = fmaxf(m[g], mb);
                const bool none = mn == -__builtin_inff();  // no key allowed yet for this query
                const float alpha = m[g] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m[g] - mn);
                l[g] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[g][db][r] *= alpha;
                m[g] = mn;
                nmu[g] = none ? __builtin_inff() : -mn;
                ps = attn_weights<TI>(s[g], pf[g], a.scale_log2, none ? 0.0f : -mn);  // no key allowed: every weight 0
            }
            l[g] += ps;
        }
#pragma unroll
        for (int t = 0; t < PT; ++t)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 vf = frag_from_rtile<D, BKV>(vt, 32 * db, 16 * t, lane);
#pragma unroll
                for (int g = 0; g < QG; ++g) o[g][db] = Mfma<TI>::run(vf, pf[g][t], o[g][db]);
            }
    };

    // A whole key block; each branch of the mask test gets its own copy
    // (sharing the score products ahead of the branch raised the register
    // count from 164 to 220).
    auto block = [&](auto mask_tag, const char *__restrict__ kt, const char *__restrict__ vt,
                     int kv0) __attribute__((always_inline)) {
        f32x16 sc[QG][SB];
        qk(kt, sc);
        softmax_pv(mask_tag, sc, vt, kv0);
    };

    // One barrier per key block. (Issuing the next block's score products
    // before this block's softmax -- a software pipeline -- needs a second
    // score register set and a deeper ring: at 190-196 registers, two waves
    // per SIMD, with MFMA/VALU interleaving hints, it measured 1-5% slower
    // than this loop at 156 registers and three waves per SIMD.)
    // The stage pointers never alias the stage being filled (restrict keeps
    // the compiler from waiting on those loads before reading these).
    const int last_q = wq0 + 32 * QG - 1;  // causal: blocks past it add nothing for this wave
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(std::true_type{}, lds + s * STAGE, s * BKV);
    int cur = 0;
    // Block kb: wait for it, synchronise, queue block kb+S-1, then compute.
    auto step = [&](auto mask_tag, int kb) __attribute__((always_inline)) {
        wait_vmcnt<(S - 2) * LOADS>();  // block kb has landed (this wave's loads)
        stage_barrier();                // ... everyone's; and everyone is done with block kb-1
        const int fill = cur == 0 ? S - 1 : cur - 1;
        issue(std::true_type{}, lds + fill * STAGE, (kb + S - 1) * BKV);
        const int kv0 = kb * BKV;
        const char *kt = lds + cur * STAGE;
        if (!CAUSAL || kv0 <= last_q) block(mask_tag, kt, kt + K_BYTES, kv0);
        cur = cur + 1 == S ? 0 : cur + 1;
    };
    // The blocks that need no mask (every key inside seq_kv and, causal, at
    // or before this wave's first query) come first, in a loop of their own:
    // with a single path through the loop, O stays in the same registers
    // from one block to the next (a masked and an unmasked path joining in
    // one loop made the compiler copy O between register sets every block).
    // Every wave runs one iteration, and one barrier, per block; the waves
    // of a workgroup only differ in which loop an iteration belongs to.
    const int nfree = min(nkv, (CAUSAL ? min(a.seq_kv, wq0 + 1) : a.seq_kv) / BKV);
    int kb = 0;
    // The unmasked blocks S at a time: block kb + u lives in stage u, so
    // every stage address is a compile-time offset and the fragment reads
    // need no per-block address arithmetic (measured +2-3 % at head_dim 64,
    // +4 % at 128). The block it queues lies inside seq_kv (the loop's
    // condition), so its loads skip the key test.
    auto step_at = [&](auto u_tag, int kb) __attribute__((always_inline)) {
        constexpr int U = decltype(u_tag)::value;
        wait_vmcnt<(S - 2) * LOADS>();
        stage_barrier();
        issue(std::false_type{}, lds + ((U + S - 1) % S) * STAGE, (kb + S - 1) * BKV);
        const int kv0 = kb * BKV;
        if (!CAUSAL || kv0 <= last_q) block(std::false_type{}, lds + U * STAGE, lds + U * STAGE + K_BYTES, kv0);
    };
    static_assert(S == 2 || S == 3, "the unrolled loop covers two or three stages");
    for (; kb + S <= nfree && (kb + 2 * S - 1) * BKV <= a.seq_kv; kb += S) {
        step_at(std::integral_constant<int, 0>{}, kb);
        step_at(std::integral_constant<int, 1>{}, kb + 1);
        if constexpr (S == 3) step_at(std::integral_constant<int, 2>{}, kb + 2);
    }
    cur = kb % S;
    for (; kb < nfree; ++kb) step(std::false_type{}, kb);
    for (; kb < nkv; ++kb) step(std::true_type{}, kb);
    wait_vmcnt<0>();  // the trailing out-of-range loads land before the workgroup exits

    // O = O^T / l (lane l holds query my_q[g], head_dim rows 32db + 8*(r/4) + 4*(l/32) + r%4)
    char *Op = static_cast<char *>(a.O);
    const int es = a.out_dtype == DG_F32 ? 4 : 2;
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const float lt = l[g] + __shfl_xor(l[g], 32);
        if (my_q[g] >= a.seq_q) continue;
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int64_t orow = ((int64_t)b * a.ob + (int64_t)h * a.oh + (int64_t)my_q[g] * a.os) * es;
        const bool vec = (((uintptr_t)Op + orow) % (uintptr_t)(4 * es)) == 0;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * db + 8 * r4 + 4 * half;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = o[g][db][4 * r4 + e] * inv;
                char *p = Op + orow + (int64_t)d0 * es;
                if (a.out_dtype == DG_F32) store4_t<DG_F32>(p, vec, 4, 1, y);
                else if (a.out_dtype == DG_BF16) store4_t<DG_BF16>(p, vec, 4, 1, y);
                else store4_t<DG_F16>(p, vec, 4, 1, y);
            }
        if (a.lse && half == 0)
            a.lse[((int64_t)b * a.heads + h) * a.seq_q + my_q[g]] =
                lt > 0.0f ? (m[g] + __log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
    }
}

template <typename TI, int D, bool CAUSAL>
static void launch_t(const AttnArgs &a, hipStream_t s) {
    const unsigned groups = (unsigned)a.batch * (unsigned)a.heads * (unsigned)a.q_blocks;
    hipLaunchKernelGGL((attn_fwd<TI, D, CAUSAL>), dim3(groups), dim3(256), 0, s, a);
}

template <typename TI, int D>
static void launch_d(const AttnArgs &a, hipStream_t s) {
    if (a.causal) launch_t<TI, D, true>(a, s);
    else launch_t<TI, D, false>(a, s);
}

hipError_t launch_attention(const AttnArgs &a, int in_dtype, int head_dim, hipStream_t s) {
    if (in_dtype != DG_BF16 && in_dtype != DG_F16) return hipErrorInvalidValue;
    const bool bf = in_dtype == DG_BF16;
    if (head_dim == 64) bf ? launch_d<BF16, 64>(a, s) : launch_d<F16, 64>(a, s);
    else if (head_dim == 128) bf ? launch_d<BF16, 128>(a, s) : launch_d<F16, 128>(a, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dg
