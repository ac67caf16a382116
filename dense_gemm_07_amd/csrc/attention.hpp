// Internal declarations of the attention forward kernel. Not part of the C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Q, K, V, O are [batch][heads][seq][head_dim] with element strides
// (batch, head, seq) and a unit stride along head_dim; lse (may be NULL) is
// fp32 [batch][heads][seq_q], contiguous.
struct AttnArgs {
    const void *Q, *K, *V;
    void *O;
    float *lse;
    int32_t batch, heads, seq_q, seq_kv;
    int64_t qb, qh, qs, kb, kh, ks, vb, vh, vs, ob, oh, os;
    float scale_log2;   // softmax scale times log2(e): the kernel exponentiates with exp2
    int32_t out_dtype;  // dg_dtype of O
    int32_t q_blocks;   // query blocks per (batch, head)
    int32_t causal;
    int32_t num_xcd;    // XCDs of the device (workgroups are dealt to them round-robin)
};

// One 32-query group per wave measured best: two groups (sharing each K/V
// fragment read) need 256+ registers, one wave per SIMD, and ran 19% slower.
constexpr int kAttnQueryGroups = 1;  // 32-query groups per wave
constexpr int kAttnBlockQ = 128;     // queries per workgroup (4 waves x groups x 32)
constexpr int kAttnBlockKV = 64;     // keys per step
constexpr int kAttnStages = 3;       // most K/V blocks in the LDS ring (head_dim 64)
// The largest sum of one lane's weights in a key block that leaves the
// reference max where it is: every weight then stays <= 2^8, well inside the
// range of fp32 sums and of the 16-bit weights fed to the second product.
constexpr float kAttnSumLimit = 256.0f;

// K/V blocks in the LDS ring for a head_dim: 3 x 16 KiB at 64; 2 x 32 KiB at
// 128 (two workgroups per CU instead of one).
constexpr int attn_stages(int head_dim) { return head_dim <= 64 ? 3 : 2; }

// Launches the kernel for an input dtype / head_dim pair; hipErrorInvalidValue
// if none is compiled.
hipError_t launch_attention(const AttnArgs &a, int in_dtype, int head_dim, hipStream_t s);

}  // namespace dg
