// Host side of the dense GEMM library: argument validation, the kernel
// registry, config selection (cache, then heuristic), the autotuner and the
// config cache. Every public symbol is declared in include/dg.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cinttypes>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "attention.hpp"
#include "dg.h"
#include "dg_internal.hpp"

namespace dg {
namespace {

thread_local std::string g_last_error;

dg_status fail(dg_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool log_enabled() {
    static const bool on = [] {
        const char *v = getenv("DG_LOG");
        return v && *v && strcmp(v, "0") != 0;
    }();
    return on;
}

int elem_size(int dt) { return dt == DG_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == DG_F32 || dt == DG_F16 || dt == DG_BF16; }
const char *dtype_name(int dt) { return dt == DG_F32 ? "f32" : dt == DG_F16 ? "f16" : dt == DG_BF16 ? "bf16" : "?"; }

// Fused epilogue of dg_gemm_ex (the defaults are a plain store).
struct Epi {
    float alpha = 1.0f, beta = 0.0f;
    const void *R = nullptr;  // residual; resolved to C when beta != 0 and none is given
    int r_dtype = DG_F32;
    int64_t srm = 0, srn = 0;
    const void *bias = nullptr;
    int bias_dtype = DG_F32;
    int per_row = 0;
    int64_t sbias = 0;
    int act = DG_ACT_NONE;
    bool general() const { return alpha != 1.0f || beta != 0.0f || bias != nullptr || act != DG_ACT_NONE; }
};

struct Problem {
    int64_t M, N, K;
    const void *A, *B;
    const void *C;
    int64_t sam, sak, sbk, sbn, scm, scn;
    int in, out;
    int64_t batch = 1;  // products of this shape
    int64_t bsa = 0, bsb = 0, bsc = 0, bsr = 0, bsbias = 0;
    Epi epi;
};

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// A 2D strided view with extents e1, e2 >= 2 and strides s1, s2 >= 1 maps two
// distinct index pairs to one element iff di*s1 == dj*s2 has a solution with
// |di| < e1, |dj| < e2, (di, dj) != 0. The smallest one is di = s2/g,
// dj = s1/g with g = gcd(s1, s2).
bool injective_2d(int64_t e1, int64_t s1, int64_t e2, int64_t s2) {
    if (e1 <= 1 || e2 <= 1) return true;
    const int64_t g = gcd64(s1, s2);
    return !(s2 / g < e1 && s1 / g < e2);
}

// Spans and stride products below are formed in 128 bits: strides are
// arbitrary int64 values.
typedef __int128 i128;

// Element span of a strided view: (e1-1)*s1 + (e2-1)*s2 + 1 (extents >= 1).
i128 span2(int64_t e1, int64_t s1, int64_t e2, int64_t s2) {
    return (i128)(e1 - 1) * s1 + (i128)(e2 - 1) * s2 + 1;
}

// Sufficient condition for a strided view to be injective: sorted by stride,
// every stride is at least the span of the dimensions with smaller strides.
bool nested(std::vector<std::pair<int64_t, int64_t>> dims) {  // (extent, stride)
    std::sort(dims.begin(), dims.end(), [](const auto &a, const auto &b) { return a.second < b.second; });
    i128 span = 1;
    for (const auto &d : dims) {
        if (d.first <= 1) continue;
        if ((i128)d.second < span) return false;
        span += (i128)(d.first - 1) * d.second;
    }
    return true;
}

// Distinct products of a batch write distinct elements of C.
bool batch_disjoint(const Problem &p) {
    if (p.batch <= 1) return true;
    if ((i128)p.bsc >= span2(p.M, p.scm, p.N, p.scn)) return true;
    return nested({{p.M, p.scm}, {p.N, p.scn}, {p.batch, p.bsc}});
}

// Byte range [lo, hi) that a strided batch of M x N views touches.
std::pair<i128, i128> byte_span(const void *base, int64_t batch, int64_t bs, int64_t M, int64_t sm, int64_t N,
                                int64_t sn, int es) {
    const i128 elems = (i128)(batch - 1) * bs + (i128)(M - 1) * sm + (i128)(N - 1) * sn + 1;
    const i128 lo = (i128)(uintptr_t)base;
    return {lo, lo + elems * es};
}

// The residual is C's own view: same address, dtype, strides and batch stride.
bool same_view_as_c(const Problem &p) {
    const Epi &e = p.epi;
    return e.R == p.C && e.r_dtype == p.out && e.srm == p.scm && e.srn == p.scn && (p.batch <= 1 || p.bsr == p.bsc);
}

bool spans_overlap(const Problem &p) {
    const Epi &e = p.epi;
    const int64_t nb = p.batch < 1 ? 1 : p.batch;
    const auto c = byte_span(p.C, nb, p.bsc, p.M, p.scm, p.N, p.scn, elem_size(p.out));
    const auto r = byte_span(e.R, nb, p.bsr, p.M, e.srm, p.N, e.srn, elem_size(e.r_dtype));
    return c.first < r.second && r.first < c.second;
}

dg_status validate_ex(const Problem &p) {
    const bool c_used = p.M > 0 && p.N > 0 && p.batch > 0;
    if (p.batch < 0) return fail(DG_ERR_INVALID_VALUE, "negative batch count");
    if (p.batch > INT32_MAX) return fail(DG_ERR_UNSUPPORTED, "batch count above 2^31 - 1");
    if (p.bsa < 0 || p.bsb < 0 || p.bsc < 0 || p.bsr < 0 || p.bsbias < 0)
        return fail(DG_ERR_INVALID_VALUE, "negative batch stride");
    if (c_used && !batch_disjoint(p))
        return fail(DG_ERR_INVALID_VALUE, "batch stride %" PRId64 " makes the C matrices of the batch overlap", p.bsc);
    const Epi &e = p.epi;
    if (e.act != DG_ACT_NONE && e.act != DG_ACT_RELU && e.act != DG_ACT_GELU)
        return fail(DG_ERR_INVALID_VALUE, "unknown activation %d", e.act);
    if (e.beta != 0.0f && c_used) {
        if (!e.R) return fail(DG_ERR_INVALID_VALUE, "residual is NULL");
        if (!dtype_ok(e.r_dtype)) return fail(DG_ERR_INVALID_VALUE, "unknown residual dtype %d", e.r_dtype);
        if (e.srm < 0 || e.srn < 0) return fail(DG_ERR_INVALID_VALUE, "negative residual stride");
        if ((uintptr_t)e.R % (uintptr_t)elem_size(e.r_dtype))
            return fail(DG_ERR_INVALID_VALUE, "residual not aligned to its element size");
        // A residual that shares memory with C must be C itself, element for
        // element (the in-place C = alpha*AB + beta*C): each workgroup then
        // reads only the elements it writes. Any other overlap would let one
        // workgroup read what another tile's workgroup is writing.
        if (p.C && !same_view_as_c(p) && spans_overlap(p))
            return fail(DG_ERR_INVALID_VALUE,
                        "residual overlaps C without being C (same pointer, dtype, strides and batch stride)");
    }
    if (e.bias && c_used) {
        if (!dtype_ok(e.bias_dtype)) return fail(DG_ERR_INVALID_VALUE, "unknown bias dtype %d", e.bias_dtype);
        if (e.sbias < 0) return fail(DG_ERR_INVALID_VALUE, "negative bias stride");
        if ((uintptr_t)e.bias % (uintptr_t)elem_size(e.bias_dtype))
            return fail(DG_ERR_INVALID_VALUE, "bias not aligned to its element size");
    }
    return DG_OK;
}

dg_status validate(const Problem &p) {
    if (!dtype_ok(p.in)) return fail(DG_ERR_INVALID_VALUE, "unknown input dtype %d", p.in);
    if (!dtype_ok(p.out)) return fail(DG_ERR_INVALID_VALUE, "unknown output dtype %d", p.out);
    if (p.M < 0 || p.N < 0 || p.K < 0)
        return fail(DG_ERR_INVALID_VALUE, "negative dimension (M=%" PRId64 ", N=%" PRId64 ", K=%" PRId64 ")", p.M, p.N, p.K);
    const int64_t lim = (int64_t)1 << 30;
    if (p.M > lim || p.N > lim || p.K > lim)
        return fail(DG_ERR_UNSUPPORTED, "dimension above 2^30 (M=%" PRId64 ", N=%" PRId64 ", K=%" PRId64 ")", p.M, p.N, p.K);
    if (p.sam < 0 || p.sak < 0 || p.sbk < 0 || p.sbn < 0)
        return fail(DG_ERR_INVALID_VALUE, "negative A/B stride");
    const bool c_used = p.M > 0 && p.N > 0;
    if (c_used && (p.scm < 1 || p.scn < 1)) return fail(DG_ERR_INVALID_VALUE, "C strides must be >= 1");
    if (c_used && !injective_2d(p.M, p.scm, p.N, p.scn))
        return fail(DG_ERR_INVALID_VALUE, "C strides (%" PRId64 ", %" PRId64 ") make elements of C overlap", p.scm, p.scn);
    const bool any = p.batch != 0;  // a batch of no products reads and writes nothing
    if (any && p.M > 0 && p.K > 0 && !p.A) return fail(DG_ERR_INVALID_VALUE, "A is NULL");
    if (any && p.K > 0 && p.N > 0 && !p.B) return fail(DG_ERR_INVALID_VALUE, "B is NULL");
    if (any && c_used && !p.C) return fail(DG_ERR_INVALID_VALUE, "C is NULL");
    const uintptr_t ie = (uintptr_t)elem_size(p.in), oe = (uintptr_t)elem_size(p.out);
    if (((uintptr_t)p.A % ie) || ((uintptr_t)p.B % ie))
        return fail(DG_ERR_INVALID_VALUE, "A or B not aligned to its element size");
    if ((uintptr_t)p.C % oe) return fail(DG_ERR_INVALID_VALUE, "C not aligned to its element size");
    return validate_ex(p);
}

// ---- layout classes --------------------------------------------------------

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Load mode of an operand viewed as rows x K with strides (srow, sk), for the
// 16-bit MFMA kernels. The vector modes move 16-byte chunks (8 elements) that
// are either wholly inside the operand's view or wholly outside it, and
// address a tile with 31-bit byte offsets (the largest tile has 256 rows).
int load_mode(const void *base, int64_t rows, int64_t K, int64_t srow, int64_t sk) {
    if (!aligned16(base)) return LD_GN;
    const int64_t lim = (int64_t)1 << 30;  // elements: 2 bytes each stays below 2^31
    // The pipeline also queues up to 8 x 64 k past K (as out-of-range loads),
    // whose offsets must not wrap either: K + 512 below.
    if (sk == 1 && K % 8 == 0 && (rows <= 1 || srow % 8 == 0) && (i128)256 * srow + K + 512 < lim) return LD_KC;
    if (srow == 1 && rows % 8 == 0 && (K <= 1 || sk % 8 == 0) && (i128)(K + 512) * sk + 256 < lim) return LD_RC;
    return LD_GN;
}

int c_class(const Problem &p) { return p.scn == 1 ? 0 : p.scm == 1 ? 1 : 2; }

// ---- registry ----------------------------------------------------------------

const std::vector<KernelEntry> &registry() {
    static const std::vector<KernelEntry> reg = [] {
        std::vector<KernelEntry> r;
        register_simt(r);
        register_mfma_bf16_kc_rc(r);
        register_mfma_bf16_kc_kc(r);
        register_mfma_bf16_rc_rc(r);
        register_mfma_bf16_rc_kc(r);
        register_mfma_bf16_gn(r);
        register_mfma_bf16_unaligned(r);
        register_mfma_f16_kc_rc(r);
        register_mfma_f16_kc_kc(r);
        register_mfma_f16_rc_rc(r);
        register_mfma_f16_rc_kc(r);
        register_mfma_f16_gn(r);
        register_mfma_f16_unaligned(r);
        register_mfma_f32(r);
        return r;
    }();
    return reg;
}

bool same_kernel(const dg_config &a, const dg_config &b) {
    return a.block_m == b.block_m && a.block_n == b.block_n && a.block_k == b.block_k && a.waves == b.waves &&
           a.stages == b.stages && a.variant == b.variant;
}

// Register-staged load mode of an operand (rows x K, strides srow, sk):
// contiguous along k or along rows at any element alignment, else elements.
int staged_mode(int64_t rows, int64_t K, int64_t srow, int64_t sk) {
    if (sk == 1 || K <= 1) return LD_KU;
    if (srow == 1 || rows <= 1) return LD_RU;
    return LD_GN;
}

// Effective load modes of the MFMA kernels for a problem. Both operands in a
// 16-byte vector layout: the direct-to-LDS kernel. Otherwise the
// register-staged kernel: contiguous operands keep 16-byte loads at any
// alignment; an operand with no unit stride makes both use element loads.
// fp32 operands on the fp32 matrix-core kernel: 16-byte chunks of 4 floats
// along k (K % 4 == 0) or along the rows (rows % 4 == 0), else elements.
int f32_mode(const void *base, int64_t rows, int64_t K, int64_t srow, int64_t sk) {
    if (!aligned16(base)) return LD_GN;
    if (sk == 1 && K % 4 == 0 && (rows <= 1 || srow % 4 == 0)) return LD_KC;
    if (srow == 1 && rows % 4 == 0 && (K <= 1 || sk % 4 == 0)) return LD_RC;
    return LD_GN;
}

std::pair<int, int> mfma_modes(const Problem &p) {
    if (p.in == DG_F32) {
        const bool a_vec = p.batch <= 1 || p.bsa % 4 == 0;
        const bool b_vec = p.batch <= 1 || p.bsb % 4 == 0;
        return {a_vec ? f32_mode(p.A, p.M, p.K, p.sam, p.sak) : LD_GN,
                b_vec ? f32_mode(p.B, p.N, p.K, p.sbn, p.sbk) : LD_GN};
    }
    // Every product of a batch starts 16-byte aligned iff the first does and
    // the batch stride is a multiple of 8 elements.
    const bool a_vec = p.batch <= 1 || p.bsa % 8 == 0;
    const bool b_vec = p.batch <= 1 || p.bsb % 8 == 0;
    const int la = a_vec ? load_mode(p.A, p.M, p.K, p.sam, p.sak) : LD_GN;
    const int lb = b_vec ? load_mode(p.B, p.N, p.K, p.sbn, p.sbk) : LD_GN;
    if (la != LD_GN && lb != LD_GN) return {la, lb};
    const int sa = staged_mode(p.M, p.K, p.sam, p.sak);
    const int sb = staged_mode(p.N, p.K, p.sbn, p.sbk);
    if (sa == LD_GN || sb == LD_GN) return {LD_GN, LD_GN};
    // The contiguous register-staged loads fetch every chunk as 16 bytes from
    // inside the operand, clamped at its edges: a k-contiguous operand needs
    // K >= 8, a row-contiguous one at least 8 rows.
    if ((sa == LD_KU || sb == LD_KU) && p.K < 8) return {LD_GN, LD_GN};
    if ((sa == LD_RU && p.M < 8) || (sb == LD_RU && p.N < 8)) return {LD_GN, LD_GN};
    return {sa, sb};
}

bool register_staged(int la) { return la == LD_KU || la == LD_RU || la == LD_GN; }

// Both operands of a 16-bit problem in the direct-to-LDS kernel's layouts.
bool direct_modes(const Problem &p) {
    if (p.in == DG_F32) return false;
    const auto m = mfma_modes(p);
    return (m.first == LD_KC || m.first == LD_RC) && (m.second == LD_KC || m.second == LD_RC);
}

// Both operands of a 16-bit problem contiguous but off 16-byte alignment
// (the register-staged kernels' 16-byte loads).
bool staged_modes(const Problem &p) {
    if (p.in == DG_F32) return false;
    const auto m = mfma_modes(p);
    return (m.first == LD_KU || m.first == LD_RU) && (m.second == LD_KU || m.second == LD_RU);
}

// The register-staged MFMA kernel always double-buffers: for a problem that
// needs it, a config's `stages` is not part of the match.
const KernelEntry *find_kernel(const dg_config &cfg, const Problem &p) {
    int la = -1, lb = -1;
    if (cfg.variant == DG_VARIANT_MFMA) std::tie(la, lb) = mfma_modes(p);
    for (const auto &e : registry()) {
        dg_config want = cfg;
        if (cfg.variant == DG_VARIANT_MFMA && register_staged(la)) want.stages = e.cfg.stages;
        if (!same_kernel(e.cfg, want)) continue;
        if (e.in_dtype != p.in) continue;
        if (e.out_dtype != -1 && e.out_dtype != p.out) continue;
        if (e.load_a != -1 && e.load_a != la) continue;
        if (e.load_b != -1 && e.load_b != lb) continue;
        return &e;
    }
    return nullptr;
}

// Distinct kernel shapes (one per tile config) usable for a dtype pair.
std::vector<dg_config> kernel_shapes(int in, int out) {
    std::vector<dg_config> shapes;
    for (const auto &e : registry()) {
        if (e.in_dtype != in || (e.out_dtype != -1 && e.out_dtype != out)) continue;
        if (in != DG_F32 && e.cfg.variant == DG_VARIANT_SIMT) continue;  // matrix cores for 16-bit inputs
        bool seen = false;
        for (const auto &s : shapes) seen = seen || same_kernel(s, e.cfg);
        if (!seen) shapes.push_back(e.cfg);
    }
    return shapes;
}

const int kGroups[] = {1, 4, 8, 16};

std::vector<dg_config> candidates(int in, int out) {
    std::vector<dg_config> c;
    for (const auto &s : kernel_shapes(in, out))
        for (int xcd = 1; xcd >= 0; --xcd)
            for (int g : kGroups) {
                dg_config x = s;
                x.group_m = g;
                x.xcd_remap = xcd;
                c.push_back(x);
            }
    return c;
}

// ---- device facts ------------------------------------------------------------

struct DeviceInfo {
    int cus = 256;
    int num_xcd = 8;
};

std::mutex g_dev_mu;
std::map<int, DeviceInfo> g_dev;

DeviceInfo device_info() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return DeviceInfo{};
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = g_dev.find(dev);
    if (it != g_dev.end()) return it->second;
    DeviceInfo d;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
        d.cus = cus;
        d.num_xcd = std::max(1, cus / 32);  // CDNA4: 32 CUs per XCD
    } else {
        (void)hipGetLastError();
    }
    g_dev[dev] = d;
    return d;
}

// ---- heuristic ---------------------------------------------------------------

// ---- split-K plan ------------------------------------------------------------

// K ranges of a config: ceil(K / k_splits) rounded up to whole K slices.
struct SplitPlan {
    int splits;
    int k_chunk;
};

SplitPlan split_plan(int64_t K, const dg_config &cfg) {
    const int want = cfg.k_splits < 1 ? 1 : cfg.k_splits;
    if (want <= 1 || K <= cfg.block_k) return {1, (int)K};
    const int64_t per = (K + want - 1) / want;
    const int64_t chunk = (per + cfg.block_k - 1) / cfg.block_k * cfg.block_k;
    return {(int)((K + chunk - 1) / chunk), (int)chunk};
}

// Workspace of a split launch: one fp32 partial tile per (product, tile,
// range). Nothing in it needs initialising (every partial is written before
// it is read, by an earlier kernel on the same stream).
struct WsLayout {
    int64_t total;  // bytes; < 0: does not fit in int64
};

WsLayout ws_layout(int64_t M, int64_t N, int64_t batch, const dg_config &cfg, int splits) {
    if (splits <= 1 || M == 0 || N == 0 || batch == 0) return {0};
    const i128 tiles = (i128)((M + cfg.block_m - 1) / cfg.block_m) * ((N + cfg.block_n - 1) / cfg.block_n) * batch;
    const i128 total = tiles * splits * cfg.block_m * cfg.block_n * 4;
    if (total > (i128)INT64_MAX) return {-1};
    return {(int64_t)total};
}

// ---- stream-K plan -----------------------------------------------------------

// One workgroup per CU (every rank resident at once), at most two per tile.
// The ranks share out the K steps of the last, partial round of G tiles
// together with one whole round before it, so each rank takes between one and
// two tiles' steps and a tile is cut into at most three pieces (its owner
// reads at most two partials); with fewer tiles than CUs, all of them.
struct SkPlan {
    int groups, tiles, iters, base, extra;
};

int sk_groups() { return device_info().cus; }

// Stream-K workspace: the flags, then one partial tile per rank (sized for
// one rank per CU).
WsLayout sk_layout(int64_t M, int64_t N, int64_t batch, const dg_config &cfg) {
    if (M == 0 || N == 0 || batch == 0) return {0};
    const int G = sk_groups();
    return {sk_flag_bytes(G) + (int64_t)G * cfg.block_m * cfg.block_n * 4};
}

// Workspace a config needs for a problem (0: none).
WsLayout ws_need(int64_t M, int64_t N, int64_t K, int64_t batch, const dg_config &cfg) {
    if (cfg.k_splits == DG_STREAM_K) return sk_layout(M, N, batch, cfg);
    return ws_layout(M, N, batch, cfg, split_plan(K, cfg).splits);
}

// false: the shared K steps do not fit in int32 (the kernel's step numbers).
bool sk_plan(int64_t total_tiles, int64_t K, const dg_config &cfg, SkPlan &out) {
    const int G = (int)std::max<int64_t>(1, std::min<int64_t>(sk_groups(), 2 * total_tiles));
    const int64_t iters = (K + cfg.block_k - 1) / cfg.block_k;
    const int64_t rem = total_tiles % G;
    int64_t shared = total_tiles <= G ? total_tiles : (rem == 0 ? 0 : rem + G);
    if (iters == 0) shared = 0;
    const int64_t S = shared * iters;
    if (S >= ((int64_t)1 << 31) || iters >= ((int64_t)1 << 31)) return false;
    out = SkPlan{G, (int)shared, (int)iters, (int)(S / G), (int)(S % G)};
    return true;
}

// Launch epochs: a stream-K flag reads as raised only with this launch's
// value. Starts at a per-process value, never 0.
uint32_t next_epoch() {
    static std::atomic<uint32_t> epoch{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() |
                                       1u};
    uint32_t e = epoch.fetch_add(1) + 1;
    if (e == 0) e = epoch.fetch_add(1) + 1;
    return e;
}

dg_config heuristic(const Problem &p, int cus, int64_t ws_bytes) {
    const auto shapes = kernel_shapes(p.in, p.out);
    const int64_t nb = p.batch < 1 ? 1 : p.batch;
    dg_config best{};
    bool have = false;
    if (p.in == DG_F32) {
        // fp32 inputs: the fp32 matrix-core kernel, 128x128 when that gives a
        // tile per CU, else 64x64 (measured on MI355X: 64x64 beats the scalar
        // kernel's tiles from 64^3 up, 1.7x at 128^3, 2.2x at 512^3); tiny
        // problems (C within two 32x32 tiles, e.g. 26^3, where the two tie)
        // keep the scalar kernel's 32x32 tile.
        const bool small = p.M * p.N <= 2 * 32 * 32;
        const int64_t t128 = ((p.M + 127) / 128) * ((p.N + 127) / 128) * nb;
        const int want = t128 >= cus ? 128 : 64;
        for (const auto &s : shapes) {
            if (small ? (s.variant == DG_VARIANT_SIMT && s.block_m == 32)
                      : (s.variant == DG_VARIANT_MFMA && s.block_m == want && find_kernel(s, p))) {
                best = s;
                have = true;
                break;
            }
        }
    } else if (direct_modes(p) || staged_modes(p)) {
        // The tile shape with the least estimated time, rounds x work per
        // workgroup / its rate. A round is one workgroup per slot (CUs x
        // workgroups that fit per CU); the rates are per CU, relative to the
        // 256x256 tile, fitted to kernel traces on MI355X (bf16, 1536^3 to
        // 5120^3). Direct kernel, at 3584^3: the 196 tiles of 256x256 took
        // 77 us, 256x128 107 (two rounds), 128x128 at two stages 96 (two per
        // CU), at three stages 116, 64x64 141. Register-staged kernel (A one
        // element off alignment), at 3584^3: 256x256 110 us, 256x128 196,
        // 128x128 229, 64x64 229. A tile count just past a round costs a
        // whole round, so "the biggest tile that still fills the CUs" lost
        // up to 45 % (3072^3 staged: 256x128, 288 tiles, 169 us, against
        // 256x256, 144 tiles, 94 us). Problems whose operands need element
        // loads keep the rule below.
        struct Cand { int bm, bn, bk, waves, stages, per_cu; double rate; };
        static const Cand kDirect[] = {
            {256, 256, 64, 8, 2, 1, 1.00}, {128, 256, 64, 4, 2, 1, 0.72}, {256, 128, 64, 4, 2, 1, 0.72},
            {128, 128, 64, 4, 3, 1, 0.67}, {128, 128, 64, 4, 2, 2, 0.80}, {64, 64, 64, 4, 4, 2, 0.48},
        };
        // (the staged kernels take any stage count: one entry per tile)
        static const Cand kStaged[] = {
            {256, 256, 64, 8, 2, 1, 1.00}, {128, 256, 64, 4, 2, 1, 0.56}, {256, 128, 64, 4, 2, 1, 0.56},
            {128, 128, 64, 4, 2, 1, 0.48}, {64, 64, 64, 4, 2, 2, 0.42},
        };
        const bool direct = direct_modes(p);
        const Cand *cands = direct ? kDirect : kStaged;
        const int ncand = direct ? (int)(sizeof(kDirect) / sizeof(Cand)) : (int)(sizeof(kStaged) / sizeof(Cand));
        double best_t = 0.0;
        for (int i = 0; i < ncand; ++i) {
            const Cand &c = cands[i];
            dg_config s{c.bm, c.bn, c.bk, 1, c.waves, c.stages, DG_VARIANT_MFMA, 0, 1};
            if (!find_kernel(s, p)) continue;
            const int64_t tiles = ((p.M + c.bm - 1) / c.bm) * ((p.N + c.bn - 1) / c.bn) * nb;
            const int64_t slots = (int64_t)cus * c.per_cu;
            const double t = (double)((tiles + slots - 1) / slots) * (c.bm * c.bn / 65536.0) * c.per_cu / c.rate;
            if (!have || t < best_t) {
                best = s;
                best_t = t;
                have = true;
            }
        }
    } else {
        // The first registered shape (best first) that has a kernel for this
        // problem's layouts and gives at least one tile per CU; else the
        // usable shape with the most tiles, and among those the least padded
        // area (the first such in registry order).
        int64_t most = -1, area = 0;
        for (const auto &s : shapes) {
            if (!find_kernel(s, p)) continue;
            const int64_t tiles = ((p.M + s.block_m - 1) / s.block_m) * ((p.N + s.block_n - 1) / s.block_n) * nb;
            if (tiles >= cus) {
                best = s;
                have = true;
                break;
            }
            const int64_t padded = tiles * s.block_m * s.block_n;
            if (tiles > most || (tiles == most && padded < area)) {
                most = tiles;
                area = padded;
                best = s;
                have = true;
            }
        }
    }
    if (!have && !shapes.empty()) best = shapes.front();
    // Register-staged 64x64 tiles with both operands k-contiguous off
    // alignment: BK 32 when BK 64 would pad K by more than 5 % (its last
    // slice mostly zeros) and BK 32 pads less. Measured on MI355X:
    // 1000x1500x777 12.5-12.8 against 13.3-13.7 us, 512x512x777 8.50 against
    // 8.96; where BK 64 pads little (2000x3000x1555, 2.8 %) BK 32 is 11 %
    // slower, and with a row-contiguous operand it is slower at any K.
    if (best.variant == DG_VARIANT_MFMA && best.block_m == 64 && best.block_n == 64 && best.block_k == 64 &&
        p.in != DG_F32 && p.K > 0) {
        const auto modes = mfma_modes(p);
        const int64_t k64 = (p.K + 63) / 64 * 64, k32 = (p.K + 31) / 32 * 32;
        if (modes.first == LD_KU && modes.second == LD_KU && (k64 - p.K) * 20 > k64 && k32 < k64) {
            dg_config c = best;
            c.block_k = 32;
            c.stages = 2;
            if (find_kernel(c, p)) best = c;
        }
    }
    best.group_m = 8;
    best.xcd_remap = 1;
    best.k_splits = 1;
    // Split-K (measured on MI355X, 64x64 tiles): S ranges pay when the tiles
    // leave CUs idle and each range keeps >= 1024 of K, so S = CUs / tiles,
    // capped by K / 1024 and 16. When the tiles fill the CUs the second
    // kernel and the partial-tile traffic cost more than they save (even at
    // K = 8192: 2048x512x8192 takes 29.8 us unsplit, 32.4 us at S = 2).
    if (best.variant == DG_VARIANT_MFMA && ws_bytes > 0 && p.K > 0) {
        const int64_t tiles = ((p.M + best.block_m - 1) / best.block_m) * ((p.N + best.block_n - 1) / best.block_n) * nb;
        int64_t s = (int64_t)cus / std::max<int64_t>(tiles, 1);
        s = std::min<int64_t>({s, 16, p.K / 1024});
        if (s >= 2) {
            dg_config c = best;
            c.k_splits = (int32_t)s;
            const WsLayout L = ws_layout(p.M, p.N, nb, c, split_plan(p.K, c).splits);
            if (L.total >= 0 && L.total <= ws_bytes) best = c;
        }
    }
    // Stream-K is never the default: measured on MI355X it was slower than
    // the unsplit kernel on every shape tried (partial last rounds of 64x64
    // and 128x128 tiles, 1.06 to 2.25 rounds, K 777 to 4096). dg_autotune_ex
    // times it when given a workspace.
    return best;
}

// ---- cache -------------------------------------------------------------------

struct Key {
    int64_t M, N, K, batch;
    int in, out, la, lb, lc;
    bool operator<(const Key &o) const {
        return std::tie(M, N, K, batch, in, out, la, lb, lc) <
               std::tie(o.M, o.N, o.K, o.batch, o.in, o.out, o.la, o.lb, o.lc);
    }
};

std::mutex g_cache_mu;
std::map<Key, dg_config> g_cache;

Key key_of(const Problem &p) {
    Key k{p.M, p.N, p.K, p.batch, p.in, p.out, -1, -1, c_class(p)};
    std::tie(k.la, k.lb) = mfma_modes(p);
    return k;
}

bool cache_get(const Key &k, dg_config &out) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = g_cache.find(k);
    if (it == g_cache.end()) return false;
    out = it->second;
    return true;
}

void cache_put(const Key &k, const dg_config &c) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache[k] = c;
}

// ---- launch ------------------------------------------------------------------

// Enqueues a problem (all products of its batch) with one config. A split
// config needs `ws` (ws_bytes) laid out as ws_layout describes.
dg_status launch(const Problem &p, const dg_config &cfg, hipStream_t stream, void *ws = nullptr,
                 int64_t ws_bytes = 0) {
    if (p.M == 0 || p.N == 0 || p.batch == 0) return DG_OK;
    if (cfg.block_m <= 0 || cfg.block_n <= 0 || cfg.block_k <= 0)
        return fail(DG_ERR_NO_CONFIG, "config has non-positive block sizes");
    if (cfg.group_m < 1) return fail(DG_ERR_NO_CONFIG, "config group_m must be >= 1");
    if (cfg.k_splits > 1 && cfg.variant != DG_VARIANT_MFMA)
        return fail(DG_ERR_NO_CONFIG, "split-K (k_splits %d) needs an MFMA config", cfg.k_splits);
    const bool sk = cfg.k_splits == DG_STREAM_K;
    if (sk && cfg.variant != DG_VARIANT_MFMA) return fail(DG_ERR_NO_CONFIG, "stream-K needs an MFMA config");
    const KernelEntry *e = find_kernel(cfg, p);
    if (!e)
        return fail(DG_ERR_NO_CONFIG,
                    "no compiled kernel for block %dx%dx%d waves %d stages %d variant %d with %s -> %s inputs",
                    cfg.block_m, cfg.block_n, cfg.block_k, cfg.waves, cfg.stages, cfg.variant, dtype_name(p.in),
                    dtype_name(p.out));
    if (sk && !e->stream_k)
        return fail(DG_ERR_NO_CONFIG, "block %dx%dx%d with %d stages has no stream-K kernel", cfg.block_m,
                    cfg.block_n, cfg.block_k, cfg.stages);
    const int64_t gm = (p.M + cfg.block_m - 1) / cfg.block_m;
    const int64_t gn = (p.N + cfg.block_n - 1) / cfg.block_n;
    const int64_t threads = (int64_t)cfg.waves * 64;
    const SplitPlan sp = split_plan(p.K, cfg);
    SkPlan skp{};
    if (sk) {
        if (gm * gn * p.batch >= ((int64_t)1 << 31) || !sk_plan(gm * gn * p.batch, p.K, cfg, skp))
            return fail(DG_ERR_UNSUPPORTED, "too many tiles or K steps for stream-K");
        const WsLayout L = sk_layout(p.M, p.N, p.batch, cfg);
        if (!ws || ws_bytes < L.total)
            return fail(DG_ERR_INVALID_VALUE, "stream-K needs a workspace of %" PRId64 " bytes (given %" PRId64 ")",
                        L.total, ws ? ws_bytes : (int64_t)0);
        if ((uintptr_t)ws % 256) return fail(DG_ERR_INVALID_VALUE, "workspace not 256-byte aligned");
    }
    const int64_t per_product = gm * gn * sp.splits;  // workgroups
    const int64_t max_groups = std::min<int64_t>(((int64_t)1 << 31) - 1, (((int64_t)1 << 32) - 1) / threads);
    if (gm * gn >= ((int64_t)1 << 31) || per_product > max_groups)
        return fail(DG_ERR_UNSUPPORTED, "too many tiles (%" PRId64 " x %" PRId64 " x %d K ranges)", gm, gn, sp.splits);
    if (sp.splits > 1) {
        const WsLayout L = ws_layout(p.M, p.N, p.batch, cfg, sp.splits);
        if (L.total < 0) return fail(DG_ERR_UNSUPPORTED, "split-K workspace size overflows");
        if (!ws || ws_bytes < L.total)
            return fail(DG_ERR_INVALID_VALUE, "split-K with %d K ranges needs a workspace of %" PRId64
                        " bytes (given %" PRId64 ")", sp.splits, L.total, ws ? ws_bytes : (int64_t)0);
        if ((uintptr_t)ws % 256) return fail(DG_ERR_INVALID_VALUE, "workspace not 256-byte aligned");
    }
    GemmArgs g{};
    g.M = (int32_t)p.M;
    g.N = (int32_t)p.N;
    g.K = (int32_t)p.K;
    g.grid_m = (int32_t)gm;
    g.grid_n = (int32_t)gn;
    g.group_m = cfg.group_m;
    g.xcd_remap = cfg.xcd_remap;
    g.num_xcd = device_info().num_xcd;
    g.out_dtype = p.out;
    g.sam = p.sam;
    g.sak = p.sak;
    g.sbk = p.sbk;
    g.sbn = p.sbn;
    g.scm = p.scm;
    g.scn = p.scn;
    g.splits = sp.splits;
    g.k_chunk = sp.k_chunk;
    g.bsa = p.bsa;
    g.bsb = p.bsb;
    g.bsc = p.bsc;
    if (sk) {
        g.ws = static_cast<float *>(ws);
        g.sk_groups = skp.groups;
        g.sk_tiles = skp.tiles;
        g.sk_iters = skp.iters;
        g.sk_base = skp.base;
        g.sk_extra = skp.extra;
        g.sk_epoch = next_epoch();
    }
    LaunchFn reduce = nullptr;
    if (sp.splits > 1) {
        g.ws = static_cast<float *>(ws);
        reduce = split_reduce_kernel(cfg.block_m, cfg.block_n, cfg.waves);
        if (!reduce)
            return fail(DG_ERR_NO_CONFIG, "no split-K reduction kernel for block %dx%d with %d waves", cfg.block_m,
                        cfg.block_n, cfg.waves);
    }
    const Epi &ep = p.epi;
    g.epi = ep.general() ? 1 : 0;
    g.act = ep.act;
    g.alpha = ep.alpha;
    g.beta = ep.beta;
    g.srm = ep.srm;
    g.srn = ep.srn;
    g.bsr = p.bsr;
    g.r_dtype = ep.r_dtype;
    g.bias_dtype = ep.bias_dtype;
    g.sbias = ep.sbias;
    g.bsbias = p.bsbias;
    g.bias_per_row = ep.per_row;
    // Products per launch: the workgroup count of one launch stays below
    // 2^31 and its thread count below 2^32.
    const int64_t chunk = sk ? p.batch : max_groups / per_product;  // stream-K: one launch of G ranks
    const int ie = elem_size(p.in), oe = elem_size(p.out);
    for (int64_t b0 = 0; b0 < p.batch; b0 += chunk) {
        g.batch = (int32_t)std::min<int64_t>(chunk, p.batch - b0);
        g.A = static_cast<const char *>(p.A) + (intptr_t)(b0 * p.bsa * ie);
        g.B = static_cast<const char *>(p.B) + (intptr_t)(b0 * p.bsb * ie);
        g.C = static_cast<char *>(const_cast<void *>(p.C)) + (intptr_t)(b0 * p.bsc * oe);
        g.R = ep.beta != 0.0f ? static_cast<const char *>(ep.R) + (intptr_t)(b0 * p.bsr * elem_size(ep.r_dtype))
                              : nullptr;
        g.bias = ep.bias ? static_cast<const char *>(ep.bias) + (intptr_t)(b0 * p.bsbias * elem_size(ep.bias_dtype))
                         : nullptr;
        hipError_t err = e->launch(g, stream);
        if (err != hipSuccess) return fail(DG_ERR_HIP, "launch of %s failed: %s", e->name, hipGetErrorString(err));
        if (reduce) {
            err = reduce(g, stream);
            if (err != hipSuccess)
                return fail(DG_ERR_HIP, "launch of the split-K reduction failed: %s", hipGetErrorString(err));
        }
    }
    return DG_OK;
}

Problem make_problem(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                     int64_t sbk, int64_t sbn, const void *C, int64_t scm, int64_t scn, int in, int out) {
    return Problem{M, N, K, A, B, C, sam, sak, sbk, sbn, scm, scn, in, out};
}

void log_choice(const char *what, const Problem &p, const dg_config &c) {
    if (!log_enabled()) return;
    fprintf(stderr,
            "[dg] %s M=%" PRId64 " N=%" PRId64 " K=%" PRId64 " batch=%" PRId64
            " %s->%s: block %dx%dx%d waves %d stages %d variant %d group_m %d xcd %d k_splits %d\n",
            what, p.M, p.N, p.K, p.batch, dtype_name(p.in), dtype_name(p.out), c.block_m, c.block_n, c.block_k,
            c.waves, c.stages, c.variant, c.group_m, c.xcd_remap, c.k_splits);
}

// Fills in the epilogue and batch of dg_gemm_ex. A beta != 0 without a
// residual reads C itself (C's dtype, strides and batch stride).
void apply_ex(Problem &p, const dg_epilogue *ep, const dg_batch *bt) {
    if (bt) {
        p.batch = bt->count;
        p.bsa = bt->stride_a;
        p.bsb = bt->stride_b;
        p.bsc = bt->stride_c;
        p.bsr = bt->stride_r;
        p.bsbias = bt->stride_bias;
    }
    if (ep) {
        Epi &e = p.epi;
        e.alpha = ep->alpha;
        e.beta = ep->beta;
        e.act = ep->activation;
        e.bias = ep->bias;
        e.bias_dtype = ep->bias_dtype;
        e.per_row = ep->bias_per_row ? 1 : 0;
        e.sbias = ep->bias_stride;
        if (ep->beta != 0.0f) {
            if (ep->residual) {
                e.R = ep->residual;
                e.r_dtype = ep->residual_dtype;
                e.srm = ep->stride_rm;
                e.srn = ep->stride_rn;
            } else {
                e.R = p.C;
                e.r_dtype = p.out;
                e.srm = p.scm;
                e.srn = p.scn;
                p.bsr = p.bsc;
            }
        }
    }
}

// True when the epilogue reads C's own prior contents (each launch then
// changes its own input).
bool reads_c(const Problem &p) { return p.epi.beta != 0.0f && p.epi.R == p.C; }

// The library's choice for a problem: the cached config, else the heuristic.
// A cached split config runs unsplit when the call has no room for its
// workspace.
dg_config choose(const Problem &p, int64_t ws_bytes, bool *from_cache = nullptr) {
    dg_config c;
    const bool hit = cache_get(key_of(p), c);
    if (hit) {
        if (c.k_splits > 1 || c.k_splits == DG_STREAM_K) {
            const WsLayout L = ws_need(p.M, p.N, p.K, p.batch, c);
            if (L.total < 0 || L.total > ws_bytes) c.k_splits = 1;
        }
    } else {
        c = heuristic(p, device_info().cus, ws_bytes);
    }
    if (from_cache) *from_cache = hit;
    return c;
}

dg_status autotune_impl(const Problem &p, hipStream_t stream, int repeats, dg_config *chosen, float *best_ms,
                        void *ws = nullptr, int64_t ws_bytes = 0);

}  // namespace
}  // namespace dg

// ---- scratch of the allocation-free entry point ---------------------------------
// Split-K partial tiles of dg_gemm_ex_noalloc live in this array: one copy per
// GPU, created when the library's code object is loaded on that GPU and held
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[DG_NOALLOC_SCRATCH_BYTES];

namespace dg {
namespace {

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch;  // device -> address of its copy of `scratch`

// The current device's copy of `scratch` (looked up on the first call on
// that device). No allocation: the array is part of the loaded code object.
dg_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DG_ERR_HIP, "hipGetSymbolAddress of the scratch array on device %d failed: %s", dev,
                        hipGetErrorString(e));
        it = g_scratch.emplace(dev, ptr).first;
    }
    *out = it->second;
    return DG_OK;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" {

const char *dg_status_string(dg_status s) {
    switch (s) {
    case DG_OK: return "DG_OK";
    case DG_ERR_INVALID_VALUE: return "DG_ERR_INVALID_VALUE";
    case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED";
    case DG_ERR_NO_CONFIG: return "DG_ERR_NO_CONFIG";
    case DG_ERR_HIP: return "DG_ERR_HIP";
    }
    return "DG_ERR_UNKNOWN";
}

const char *dg_last_error(void) { return g_last_error.c_str(); }

dg_status dg_validate(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                      int64_t sbk, int64_t sbn, const void *C, int64_t scm, int64_t scn, dg_dtype in_dtype,
                      dg_dtype out_dtype) {
    g_last_error.clear();
    return validate(make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype));
}

dg_status dg_select_config_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak,
                              const void *B, int64_t sbk, int64_t sbn, const void *C, int64_t scm, int64_t scn,
                              dg_dtype in_dtype, dg_dtype out_dtype, const dg_batch *batch, int64_t workspace_bytes,
                              dg_config *out, int32_t *from_cache) {
    g_last_error.clear();
    if (!out) return fail(DG_ERR_INVALID_VALUE, "out is NULL");
    if (workspace_bytes < 0) return fail(DG_ERR_INVALID_VALUE, "negative workspace size");
    // NULL pointers are inspected for alignment only: stand in an aligned address.
    static const char aligned_stub[16] __attribute__((aligned(16))) = {0};
    Problem p = make_problem(M, N, K, A ? A : aligned_stub, sam, sak, B ? B : aligned_stub, sbk, sbn,
                             C ? C : aligned_stub, scm, scn, in_dtype, out_dtype);
    apply_ex(p, nullptr, batch);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    bool hit = false;
    *out = choose(p, workspace_bytes, &hit);
    if (from_cache) *from_cache = hit ? 1 : 0;
    return DG_OK;
}

dg_status dg_select_config(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                           int64_t sbk, int64_t sbn, const void *C, int64_t scm, int64_t scn, dg_dtype in_dtype,
                           dg_dtype out_dtype, dg_config *out, int32_t *from_cache) {
    return dg_select_config_ex(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype, nullptr, 0, out,
                               from_cache);
}

dg_status dg_gemm_config(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                         int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn, dg_dtype in_dtype,
                         dg_dtype out_dtype, void *stream, const dg_config *cfg) {
    g_last_error.clear();
    if (!cfg) return fail(DG_ERR_INVALID_VALUE, "cfg is NULL");
    Problem p = make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    return launch(p, *cfg, (hipStream_t)stream);
}

dg_status dg_gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                  int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn, dg_dtype in_dtype, dg_dtype out_dtype,
                  void *stream) {
    g_last_error.clear();
    Problem p = make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    if (M == 0 || N == 0) return DG_OK;
    dg_config c;
    if (!cache_get(key_of(p), c)) {
        static const bool tune_on_miss = [] {
            const char *v = getenv("DG_AUTOTUNE_ON_MISS");
            return v && strcmp(v, "1") == 0;
        }();
        if (tune_on_miss) return autotune_impl(p, (hipStream_t)stream, 0, nullptr, nullptr);
    }
    c = choose(p, 0);
    log_choice("gemm", p, c);
    return launch(p, c, (hipStream_t)stream);
}

dg_status dg_gemm_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                     int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn, dg_dtype in_dtype,
                     dg_dtype out_dtype, void *stream, const dg_epilogue *epilogue, const dg_batch *batch,
                     const dg_config *cfg, void *workspace, int64_t workspace_bytes) {
    g_last_error.clear();
    if (workspace_bytes < 0) return fail(DG_ERR_INVALID_VALUE, "negative workspace size");
    if (!workspace) workspace_bytes = 0;
    Problem p = make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype);
    apply_ex(p, epilogue, batch);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return DG_OK;
    const dg_config c = cfg ? *cfg : choose(p, workspace_bytes);
    if (!cfg) log_choice("gemm_ex", p, c);
    return launch(p, c, (hipStream_t)stream, workspace, workspace_bytes);
}

dg_status dg_gemm_ex_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak,
                             const void *B, int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn,
                             dg_dtype in_dtype, dg_dtype out_dtype, void *stream, const dg_epilogue *epilogue,
                             const dg_batch *batch, const dg_config *cfg) {
    g_last_error.clear();
    Problem p = make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype);
    apply_ex(p, epilogue, batch);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return DG_OK;
    const int64_t cap = DG_NOALLOC_SCRATCH_BYTES;
    const dg_config c = cfg ? *cfg : choose(p, cap);
    if (c.k_splits > 1 || c.k_splits == DG_STREAM_K) {
        const WsLayout L = ws_need(p.M, p.N, p.K, p.batch, c);
        if (L.total < 0 || L.total > cap)
            return fail(DG_ERR_UNSUPPORTED,
                        "%s partials of this call need %" PRId64 " bytes of scratch; the allocation-free "
                        "entry point holds at most %" PRId64 " bytes",
                        c.k_splits == DG_STREAM_K ? "stream-K" : "split-K", L.total, cap);
    }
    void *ws = nullptr;
    s = scratch_address(&ws);
    if (s != DG_OK) return s;
    if (!cfg) log_choice("gemm_ex_noalloc", p, c);
    return launch(p, c, (hipStream_t)stream, ws, cap);
}

dg_status dg_attention_fwd(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_kv, int64_t head_dim,
                           const void *Q, const int64_t *q_strides, const void *K, const int64_t *k_strides,
                           const void *V, const int64_t *v_strides, void *O, const int64_t *o_strides, float *lse,
                           dg_dtype in_dtype, dg_dtype out_dtype, float scale, int32_t causal, void *stream) {
    g_last_error.clear();
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(DG_ERR_INVALID_VALUE, "unknown dtype");
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || head_dim < 0)
        return fail(DG_ERR_INVALID_VALUE, "negative size");
    const int64_t lim = (int64_t)1 << 30;
    if (seq_q >= lim || seq_kv >= lim || batch * heads >= lim)
        return fail(DG_ERR_UNSUPPORTED, "sizes too large for the attention kernel");
    if (batch == 0 || heads == 0 || seq_q == 0) return DG_OK;
    if (!q_strides || !k_strides || !v_strides || !o_strides) return fail(DG_ERR_INVALID_VALUE, "strides are NULL");
    if (!Q || !O || (seq_kv > 0 && (!K || !V))) return fail(DG_ERR_INVALID_VALUE, "a tensor pointer is NULL");
    for (const int64_t *st : {q_strides, k_strides, v_strides, o_strides})
        for (int i = 0; i < 3; ++i)
            if (st[i] < 0) return fail(DG_ERR_INVALID_VALUE, "negative stride");
    if (in_dtype == DG_F32) return fail(DG_ERR_UNSUPPORTED, "attention takes fp16 or bf16 Q, K, V");
    if (head_dim != 64 && head_dim != 128)
        return fail(DG_ERR_UNSUPPORTED, "head_dim %" PRId64 " (supported: 64, 128)", head_dim);
    // O's rows must not overlap: (batch, head, seq, dim) strides nested when sorted.
    if (!nested({{batch, o_strides[0]}, {heads, o_strides[1]}, {seq_q, o_strides[2]}, {head_dim, 1}}))
        return fail(DG_ERR_INVALID_VALUE, "O strides make its elements overlap");
    const struct {
        const void *p;
        const int64_t *st;
        const char *name;
    } ins[] = {{Q, q_strides, "Q"}, {K, k_strides, "K"}, {V, v_strides, "V"}};
    for (const auto &t : ins) {
        if (seq_kv == 0 && t.p != Q) continue;  // K and V are not read
        if (!aligned16(t.p) || t.st[0] % 8 || t.st[1] % 8 || t.st[2] % 8)
            return fail(DG_ERR_UNSUPPORTED, "%s needs a 16-byte aligned base and strides that are multiples of 8",
                        t.name);
    }
    if ((uintptr_t)O % (uintptr_t)elem_size(out_dtype)) return fail(DG_ERR_INVALID_VALUE, "O misaligned");
    // The key-block loads address one (batch, head) with 31-bit byte offsets,
    // including the blocks queued past the end.
    const i128 span = (i128)(seq_kv + kAttnStages * kAttnBlockKV) * std::max(k_strides[2], v_strides[2]) * 2;
    if (span >= ((i128)1 << 31)) return fail(DG_ERR_UNSUPPORTED, "K/V of one head span more than 2 GiB");
    const int64_t q_blocks = (seq_q + kAttnBlockQ - 1) / kAttnBlockQ;
    if (batch * heads * q_blocks >= ((int64_t)1 << 31) / 256)
        return fail(DG_ERR_UNSUPPORTED, "too many query blocks");
    AttnArgs a{};
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.lse = lse;
    a.batch = (int32_t)batch;
    a.heads = (int32_t)heads;
    a.seq_q = (int32_t)seq_q;
    a.seq_kv = (int32_t)seq_kv;
    a.qb = q_strides[0], a.qh = q_strides[1], a.qs = q_strides[2];
    a.kb = k_strides[0], a.kh = k_strides[1], a.ks = k_strides[2];
    a.vb = v_strides[0], a.vh = v_strides[1], a.vs = v_strides[2];
    a.ob = o_strides[0], a.oh = o_strides[1], a.os = o_strides[2];
    const float sc = (scale > 0.0f) ? scale : 1.0f / std::sqrt((float)head_dim);
    a.scale_log2 = sc * 1.44269504088896340736f;
    a.out_dtype = out_dtype;
    a.q_blocks = (int32_t)q_blocks;
    a.causal = causal ? 1 : 0;
    a.num_xcd = device_info().num_xcd;
    const hipError_t err = launch_attention(a, in_dtype, (int)head_dim, (hipStream_t)stream);
    if (err != hipSuccess) return fail(DG_ERR_HIP, "attention launch failed: %s", hipGetErrorString(err));
    return DG_OK;
}

dg_status dg_workspace_size(int64_t M, int64_t N, int64_t K, int64_t batch_count, const dg_config *cfg,
                            int64_t *bytes) {
    g_last_error.clear();
    if (!cfg || !bytes) return fail(DG_ERR_INVALID_VALUE, "NULL argument");
    if (M < 0 || N < 0 || K < 0 || batch_count < 0) return fail(DG_ERR_INVALID_VALUE, "negative size");
    if (cfg->block_m <= 0 || cfg->block_n <= 0 || cfg->block_k <= 0)
        return fail(DG_ERR_INVALID_VALUE, "non-positive block size");
    const WsLayout L = ws_need(M, N, K, batch_count, *cfg);
    if (L.total < 0) return fail(DG_ERR_UNSUPPORTED, "workspace size overflows");
    *bytes = L.total;
    return DG_OK;
}

dg_status dg_autotune_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                         int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn, dg_dtype in_dtype,
                         dg_dtype out_dtype, void *stream, const dg_epilogue *epilogue, const dg_batch *batch,
                         void *workspace, int64_t workspace_bytes, int32_t repeats, dg_config *chosen,
                         float *best_ms) {
    g_last_error.clear();
    if (workspace_bytes < 0) return fail(DG_ERR_INVALID_VALUE, "negative workspace size");
    if (!workspace) workspace_bytes = 0;
    Problem p = make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype);
    apply_ex(p, epilogue, batch);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    if (reads_c(p) && p.M > 0 && p.N > 0 && p.batch > 0)
        return fail(DG_ERR_INVALID_VALUE, "cannot autotune an epilogue that reads C (every trial launch changes C)");
    return autotune_impl(p, (hipStream_t)stream, repeats, chosen, best_ms, workspace, workspace_bytes);
}

dg_status dg_autotune(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak, const void *B,
                      int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn, dg_dtype in_dtype,
                      dg_dtype out_dtype, void *stream, int32_t repeats, dg_config *chosen, float *best_ms) {
    g_last_error.clear();
    Problem p = make_problem(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype);
    dg_status s = validate(p);
    if (s != DG_OK) return s;
    return autotune_impl(p, (hipStream_t)stream, repeats, chosen, best_ms);
}

int32_t dg_num_candidates(dg_dtype in_dtype, dg_dtype out_dtype) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return 0;
    return (int32_t)candidates(in_dtype, out_dtype).size();
}

dg_status dg_get_candidate(int32_t i, dg_dtype in_dtype, dg_dtype out_dtype, dg_config *out) {
    g_last_error.clear();
    if (!out) return fail(DG_ERR_INVALID_VALUE, "out is NULL");
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(DG_ERR_INVALID_VALUE, "unknown dtype");
    const auto c = candidates(in_dtype, out_dtype);
    if (i < 0 || (size_t)i >= c.size()) return fail(DG_ERR_INVALID_VALUE, "candidate index %d out of range", i);
    *out = c[(size_t)i];
    return DG_OK;
}

dg_status dg_tile_coords(int32_t grid_m, int32_t grid_n, int32_t group_m, int32_t xcd_remap, int32_t num_xcd,
                         int32_t wg, int32_t *pid_m, int32_t *pid_n) {
    g_last_error.clear();
    if (grid_m <= 0 || grid_n <= 0 || group_m <= 0 || num_xcd <= 0)
        return fail(DG_ERR_INVALID_VALUE, "grid, group and XCD counts must be positive");
    if ((int64_t)grid_m * grid_n >= ((int64_t)1 << 31)) return fail(DG_ERR_INVALID_VALUE, "grid too large");
    if (wg < 0 || (int64_t)wg >= (int64_t)grid_m * grid_n) return fail(DG_ERR_INVALID_VALUE, "workgroup id out of range");
    if (!pid_m || !pid_n) return fail(DG_ERR_INVALID_VALUE, "output pointer is NULL");
    int pm, pn;
    tile_coords(wg, grid_m, grid_n, group_m, xcd_remap, num_xcd, pm, pn);
    *pid_m = pm;
    *pid_n = pn;
    return DG_OK;
}

dg_status dg_grid_shape(int64_t M, int64_t N, int64_t K, const dg_config *cfg, int64_t *grid_m, int64_t *grid_n,
                        int64_t *k_steps) {
    g_last_error.clear();
    if (!cfg || !grid_m || !grid_n || !k_steps) return fail(DG_ERR_INVALID_VALUE, "NULL argument");
    if (M < 0 || N < 0 || K < 0) return fail(DG_ERR_INVALID_VALUE, "negative dimension");
    if (cfg->block_m <= 0 || cfg->block_n <= 0 || cfg->block_k <= 0)
        return fail(DG_ERR_INVALID_VALUE, "non-positive block size");
    *grid_m = (M + cfg->block_m - 1) / cfg->block_m;
    *grid_n = (N + cfg->block_n - 1) / cfg->block_n;
    *k_steps = (K + cfg->block_k - 1) / cfg->block_k;
    return DG_OK;
}

dg_status dg_cache_clear(void) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache.clear();
    return DG_OK;
}

int32_t dg_cache_size(void) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    return (int32_t)g_cache.size();
}

static const char kCacheHeader[] = "dg-config-cache 2";

dg_status dg_cache_save(const char *path) {
    g_last_error.clear();
    if (!path) return fail(DG_ERR_INVALID_VALUE, "path is NULL");
    std::map<Key, dg_config> snapshot;
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        snapshot = g_cache;
    }
    FILE *f = fopen(path, "w");
    if (!f) return fail(DG_ERR_INVALID_VALUE, "cannot open %s for writing", path);
    fprintf(f, "%s\n", kCacheHeader);
    for (const auto &kv : snapshot) {
        const Key &k = kv.first;
        const dg_config &c = kv.second;
        fprintf(f, "%" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %d %d %d %d %d  %d %d %d %d %d %d %d %d %d\n",
                k.M, k.N, k.K, k.batch, k.in, k.out, k.la, k.lb, k.lc, c.block_m, c.block_n, c.block_k, c.group_m,
                c.waves, c.stages, c.variant, c.xcd_remap, c.k_splits);
    }
    const bool ok = fclose(f) == 0;
    return ok ? DG_OK : fail(DG_ERR_INVALID_VALUE, "error writing %s", path);
}

dg_status dg_cache_load(const char *path) {
    g_last_error.clear();
    if (!path) return fail(DG_ERR_INVALID_VALUE, "path is NULL");
    FILE *f = fopen(path, "r");
    if (!f) return fail(DG_ERR_INVALID_VALUE, "cannot open %s", path);
    char line[512];
    if (!fgets(line, sizeof(line), f) || strncmp(line, kCacheHeader, sizeof(kCacheHeader) - 1) != 0) {
        fclose(f);
        return fail(DG_ERR_INVALID_VALUE, "%s is not a config cache file", path);
    }
    int bad = 0, good = 0;
    std::vector<std::pair<Key, dg_config>> entries;
    while (fgets(line, sizeof(line), f)) {
        Key k{};
        dg_config c{};
        const int n = sscanf(line,
                             "%" SCNd64 " %" SCNd64 " %" SCNd64 " %" SCNd64 " %d %d %d %d %d %d %d %d %d %d %d %d %d %d",
                             &k.M, &k.N, &k.K, &k.batch, &k.in, &k.out, &k.la, &k.lb, &k.lc, &c.block_m, &c.block_n,
                             &c.block_k, &c.group_m, &c.waves, &c.stages, &c.variant, &c.xcd_remap, &c.k_splits);
        const bool sane = n == 18 && k.M >= 0 && k.N >= 0 && k.K >= 0 && k.batch >= 0 && dtype_ok(k.in) &&
                          dtype_ok(k.out) && c.block_m > 0 && c.block_n > 0 && c.block_k > 0 && c.group_m > 0 &&
                          (c.k_splits >= 0 || c.k_splits == DG_STREAM_K);
        if (!sane) {
            ++bad;
            continue;
        }
        entries.emplace_back(k, c);
        ++good;
    }
    fclose(f);
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        for (const auto &e : entries) g_cache[e.first] = e.second;
    }
    if (bad) {
        g_last_error = std::to_string(bad) + " malformed line(s) skipped in " + path;
        if (log_enabled()) fprintf(stderr, "[dg] %s\n", g_last_error.c_str());
    }
    return DG_OK;
}

}  // extern "C"

namespace dg {
namespace {

// Split counts the autotuner tries when a workspace is given and the tiles
// of a shape do not fill the GPU.
const int kSplits[] = {2, 4, 8, 16};

dg_status autotune_impl(const Problem &p, hipStream_t stream, int repeats, dg_config *chosen, float *best_ms,
                        void *ws, int64_t ws_bytes) {
    if (repeats <= 0) repeats = 10;
    if (p.M == 0 || p.N == 0 || p.batch == 0) {
        dg_config c = heuristic(p, device_info().cus, ws_bytes);
        if (chosen) *chosen = c;
        if (best_ms) *best_ms = 0.0f;
        return DG_OK;
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return fail(DG_ERR_HIP, "hipEventCreate failed");
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return fail(DG_ERR_HIP, "hipEventCreate failed");
    }
    std::vector<dg_config> cands;
    const int cus = device_info().cus;
    for (const auto &c : candidates(p.in, p.out)) {
        cands.push_back(c);
        if (c.variant != DG_VARIANT_MFMA || ws_bytes <= 0) continue;
        const int64_t tiles = ((p.M + c.block_m - 1) / c.block_m) * ((p.N + c.block_n - 1) / c.block_n) * p.batch;
        if (tiles > cus && tiles % cus != 0) {
            // a partial last round: stream-K shares it out
            dg_config x = c;
            x.k_splits = DG_STREAM_K;
            const KernelEntry *e = find_kernel(x, p);
            const WsLayout L = sk_layout(p.M, p.N, p.batch, x);
            SkPlan plan;
            if (e && e->stream_k && L.total <= ws_bytes && sk_plan(tiles, p.K, x, plan)) cands.push_back(x);
        }
        if (tiles >= cus) continue;
        for (int sk : kSplits) {
            dg_config x = c;
            x.k_splits = sk;
            const int used = split_plan(p.K, x).splits;
            if (used < sk && sk != kSplits[0]) continue;  // same ranges as a smaller count
            if (used < 2) continue;
            const WsLayout L = ws_layout(p.M, p.N, p.batch, x, used);
            if (L.total >= 0 && L.total <= ws_bytes) cands.push_back(x);
        }
    }
    dg_config best{};
    float best_t = 0.0f;
    bool have = false;
    dg_status st = DG_OK;
    std::vector<float> times;
    for (const auto &c : cands) {
        if (!find_kernel(c, p)) continue;
        bool ok = true;
        for (int w = 0; w < 2 && ok; ++w) ok = launch(p, c, stream, ws, ws_bytes) == DG_OK;
        times.clear();
        for (int r = 0; r < repeats && ok; ++r) {
            ok = hipEventRecord(e0, stream) == hipSuccess && launch(p, c, stream, ws, ws_bytes) == DG_OK &&
                 hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
            float ms = 0.0f;
            ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
            times.push_back(ms);
        }
        if (!ok) {
            st = fail(DG_ERR_HIP, "autotune: candidate %dx%dx%d failed: %s", c.block_m, c.block_n, c.block_k,
                      g_last_error.c_str());
            break;
        }
        std::sort(times.begin(), times.end());
        const float med = times[times.size() / 2];
        if (log_enabled())
            fprintf(stderr, "[dg] autotune %dx%dx%d w%d s%d g%d xcd%d split%d: %.4f ms\n", c.block_m, c.block_n,
                    c.block_k, c.waves, c.stages, c.group_m, c.xcd_remap, c.k_splits, med);
        if (!have || med < best_t) {
            best = c;
            best_t = med;
            have = true;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != DG_OK) return st;
    if (!have) return fail(DG_ERR_UNSUPPORTED, "no candidate kernel for %s -> %s", dtype_name(p.in), dtype_name(p.out));
    cache_put(key_of(p), best);
    log_choice("autotune winner", p, best);
    st = launch(p, best, stream, ws, ws_bytes);
    if (st != DG_OK) return st;
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(DG_ERR_HIP, "hipStreamSynchronize failed");
    if (chosen) *chosen = best;
    if (best_ms) *best_ms = best_t;
    return DG_OK;
}

}  // namespace
}  // namespace dg
