// C ABI of libkvss: argument validation (host only, before any HIP call), launch planning,
// workspace carving and error reporting. The operations are declared and specified in
// include/kvss.h.

#include <float.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "kvss.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return KVSS_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(KVSS_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
using namespace kvss_plan;     // Plan, plan_splits, verify_plan, ceil_div, workgroup targets

constexpr int kMaxGamma = 31;      // speculation length limit of spec_accept
constexpr int kMaxGridYZ = 65535;  // batch and KV heads index the y / z grid dimensions
constexpr int kDraftStream = 2;    // Philox stream of the draft-token race

int check_kv(const kvss_kv* kv) {
    if (!kv) return fail(KVSS_EINVAL, "kv descriptor is NULL");
    if (kv->batch < 0) return fail(KVSS_EINVAL, "batch must be >= 0 (got %d)", kv->batch);
    if (kv->dtype != KVSS_F32 && kv->dtype != KVSS_BF16)
        return fail(KVSS_EUNSUPPORTED, "dtype %d is not KVSS_F32 or KVSS_BF16", kv->dtype);
    if (kv->head_dim != 64 && kv->head_dim != 128)
        return fail(KVSS_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", kv->head_dim);
    if (kv->block_size <= 0 || kv->block_size % 16 != 0)
        return fail(KVSS_EUNSUPPORTED, "block_size %d is not a positive multiple of 16", kv->block_size);
    if (kv->num_kv_heads <= 0) return fail(KVSS_EINVAL, "num_kv_heads must be >= 1");
    if (kv->batch > kMaxGridYZ || kv->num_kv_heads > kMaxGridYZ)
        return fail(KVSS_EUNSUPPORTED, "batch %d or num_kv_heads %d exceeds %d", kv->batch,
                    kv->num_kv_heads, kMaxGridYZ);
    if (kv->max_kv_len < 0) return fail(KVSS_EINVAL, "max_kv_len must be >= 0");
    if (kv->batch == 0) return ok();
    if (kv->max_blocks <= 0 || kv->num_blocks <= 0)
        return fail(KVSS_EINVAL, "max_blocks and num_blocks must be >= 1");
    if ((long)kv->max_kv_len > (long)kv->max_blocks * kv->block_size)
        return fail(KVSS_EINVAL, "max_kv_len %d exceeds max_blocks * block_size = %ld", kv->max_kv_len,
                    (long)kv->max_blocks * kv->block_size);
    if (!kv->k || !kv->v || !kv->block_table || !kv->kv_lens)
        return fail(KVSS_EINVAL, "kv tensors (k, v, block_table, kv_lens) must be non-NULL");
    if ((long long)kv->num_blocks * kv->num_kv_heads * kv->block_size > 0xffffffffLL)
        return fail(KVSS_EUNSUPPORTED, "cache rows num_blocks * num_kv_heads * block_size exceed 2^32 - 1");
    return ok();
}

kvss::AttnArgs attn_common(const kvss_kv* kv) {
    kvss::AttnArgs a{};
    a.k = kv->k;
    a.v = kv->v;
    a.block_table = kv->block_table;
    a.kv_lens = kv->kv_lens;
    a.B = kv->batch;
    a.Hkv = kv->num_kv_heads;
    a.D = kv->head_dim;
    a.bs = kv->block_size;
    a.max_blocks = kv->max_blocks;
    a.num_blocks = kv->num_blocks;
    a.max_kv_len = kv->max_kv_len;
    return a;
}

float scale_log2(float scale) { return (float)((double)scale * 1.4426950408889634); }

size_t partial_bytes(long rows, const Plan& p, int D) {
    return p.nsplit > 1 ? align_up((size_t)rows * p.nsplit * (D + 2) * sizeof(float)) : 0;
}

int check_heads(const kvss_kv* kv, int num_q_heads) {
    if (num_q_heads <= 0 || num_q_heads % kv->num_kv_heads != 0)
        return fail(KVSS_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                    num_q_heads, kv->num_kv_heads);
    return ok();
}

int run_attention(kvss::AttnArgs& a, const Plan& p, bool gather, int dtype, void* ws,
                  hipStream_t s) {
    a.nsplit = p.nsplit;
    a.split_len = p.split_len;
    a.part = p.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
    hipError_t e = dtype == KVSS_BF16 ? kvss::launch_attn_mfma(a, gather, s)
                                      : kvss::launch_attn_simple(a, gather, s);
    if (e != hipSuccess) return hip_status(e, "attention launch");
    if (p.nsplit > 1) {
        e = kvss::launch_merge(a.part, a.B * a.Hq * a.T, p.nsplit, a.D, a.out, a.lse, s);
        if (e != hipSuccess) return hip_status(e, "split merge launch");
    }
    return ok();
}

struct SnapLayout {
    Plan p1;
    int R, n_stride, xs_stride;
    size_t part1, rowc, scores, pooled, xs, total;
};

SnapLayout snap_layout(const kvss_kv* kv, int num_q_heads, int w, bool own_scores) {
    SnapLayout s{};
    const int G = num_q_heads / kv->num_kv_heads;
    s.R = G * w;
    // bf16 splits must fit one LDS table of block bases (kSnapTableEntries - 1 blocks).
    s.p1 = kv->dtype == KVSS_BF16
               ? plan_splits((long)kv->batch * kv->num_kv_heads, kv->max_kv_len, kMfmaUnit,
                             (long)(kvss::kSnapTableEntries - 1) * kv->block_size,
                             kSnapTargetWorkgroups)
               : plan_splits((long)kv->batch * kv->num_kv_heads, kv->max_kv_len, kSimpleUnit);
    s.n_stride = kv->max_kv_len > w ? kv->max_kv_len - w : 0;
    const size_t rows = (size_t)kv->batch * kv->num_kv_heads;
    s.part1 = align_up(rows * s.R * s.p1.nsplit * 2 * sizeof(float));
    s.rowc = align_up(rows * s.R * sizeof(float));
    s.scores = own_scores ? align_up(rows * s.n_stride * sizeof(float)) : 0;
    s.pooled = align_up(rows * s.n_stride * sizeof(float));
    // With few rows the first pass keeps its scaled scores (4 R bytes per candidate, written
    // once and read once) instead of the second pass reading K again (2 D bytes per key).
    const bool store = kv->dtype == KVSS_BF16 && s.R <= 16 && 4 * s.R < kv->head_dim;
    s.xs_stride = (s.n_stride + 3) / 4 * 4;
    s.xs = store ? align_up(rows * s.R * s.xs_stride * sizeof(float)) : 0;
    s.total = s.part1 + s.rowc + s.scores + s.pooled + s.xs;
    return s;
}

// 0 (greedy) or a finite positive temperature whose reciprocal is a finite float.
bool temperature_ok(float t) {
    return t == 0.f || (t > 0.f && isfinite(t) && 1.0 / (double)t < (double)FLT_MAX);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// ---------------------------------------------------------------------------------------
// verify_attn_full_noalloc: the same verify, with its split partials in a library-owned
// device array instead of a caller workspace, for callers that cannot allocate.

// Largest split-partial area the no-allocation verify accepts: the plan asks for about 1024
// workgroups, so [B * Hq * T, nsplit, D + 2] floats stay near 2048 * G * T * (D + 2) * 4
// bytes, ~11 MB at G * T = 20 and head_dim 128.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// One copy per GPU the library runs on, held until the process ends. In host code the name
// stands for a host-side shadow, not a device address: kernels get the per-device address
// that scratch_on_current_device() looks up.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
int scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVSS_EUNSUPPORTED, "device ordinal %d is beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(KVSS_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

extern "C" int verify_attn_full_noalloc(const kvss_kv* kv, const void* q, int num_q_heads, int T,
                                        float scale, float* out, float* lse, void* stream) {
    int rc = check_kv(kv);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (T <= 0) return fail(KVSS_EINVAL, "T (gamma + 1) must be >= 1 (got %d)", T);
    const int G = num_q_heads / kv->num_kv_heads;
    if (G * T > 32) return fail(KVSS_EUNSUPPORTED, "G * T = %d exceeds 32 query rows per KV head", G * T);
    if (!isfinite(scale)) return fail(KVSS_EINVAL, "scale must be finite");
    if (kv->batch == 0) return ok();
    if (!q || !out) return fail(KVSS_EINVAL, "q and out must be non-NULL");
    const size_t need = kvss_verify_workspace_bytes(kv, num_q_heads, T);
    if (need > kNoAllocScratchBytes)
        return fail(KVSS_EWORKSPACE,
                    "split partials of %zu bytes exceed the %zu-byte no-allocation scratch; "
                    "use verify_attn_full with a workspace", need, kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0 && (rc = scratch_on_current_device(&ws))) return rc;
    return verify_attn_full(kv, q, num_q_heads, T, scale, out, lse, ws, need, stream);
}

extern "C" {

const char* kvss_last_error(void) { return g_err.c_str(); }

int kvss_version(void) { return 1; }

size_t kvss_verify_workspace_bytes(const kvss_kv* kv, int num_q_heads, int T) {
    if (check_kv(kv) != KVSS_OK || num_q_heads <= 0 || T <= 0) return 0;
    return partial_bytes((long)kv->batch * num_q_heads * T, verify_plan(kv), kv->head_dim);
}

int verify_attn_full(const kvss_kv* kv, const void* q, int num_q_heads, int T, float scale,
                     float* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
    int rc = check_kv(kv);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (T <= 0) return fail(KVSS_EINVAL, "T (gamma + 1) must be >= 1 (got %d)", T);
    const int G = num_q_heads / kv->num_kv_heads;
    if (G * T > 32) return fail(KVSS_EUNSUPPORTED, "G * T = %d exceeds 32 query rows per KV head", G * T);
    if (!isfinite(scale)) return fail(KVSS_EINVAL, "scale must be finite");
    if (kv->batch == 0) return ok();
    if (!q || !out) return fail(KVSS_EINVAL, "q and out must be non-NULL");
    const Plan p = verify_plan(kv);
    const size_t need = partial_bytes((long)kv->batch * num_q_heads * T, p, kv->head_dim);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KVSS_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    kvss::AttnArgs a = attn_common(kv);
    a.q = q;
    a.Hq = num_q_heads;
    a.G = G;
    a.T = T;
    a.R = G * T;
    a.scale_log2 = scale_log2(scale);
    a.out = out;
    a.lse = lse;
    return run_attention(a, p, false, kv->dtype, workspace, static_cast<hipStream_t>(stream));
}

// A draft set is short (hundreds to a few thousand keys): split only until every CU holds its
// two resident single-row-tile workgroups; more splits add a merge launch and a second round.
static Plan draft_plan(const kvss_kv* kv, int k_max, int max_tail) {
    return plan_splits((long)kv->batch * kv->num_kv_heads, (long)k_max + max_tail,
                       kv->dtype == KVSS_BF16 ? kMfmaUnit : kSimpleUnit, 1L << 30,
                       kDraftTargetWorkgroups);
}

size_t kvss_draft_workspace_bytes(const kvss_kv* kv, int num_q_heads, int k_max, int max_tail) {
    if (check_kv(kv) != KVSS_OK || num_q_heads <= 0 || k_max < 0 || max_tail < 0) return 0;
    return partial_bytes((long)kv->batch * num_q_heads, draft_plan(kv, k_max, max_tail),
                         kv->head_dim);
}

int draft_attn_sparse(const kvss_kv* kv, const void* q, int num_q_heads, const int32_t* sel_idx,
                      const int32_t* sel_count, int k_max, const int32_t* tail_lo, int max_tail,
                      float scale, float* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int rc = check_kv(kv);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    const int G = num_q_heads / kv->num_kv_heads;
    if (G > 32) return fail(KVSS_EUNSUPPORTED, "G = %d exceeds 32 query rows per KV head", G);
    if (k_max < 0) return fail(KVSS_EINVAL, "k_max must be >= 0");
    if (max_tail < 0) return fail(KVSS_EINVAL, "max_tail must be >= 0");
    if (!isfinite(scale)) return fail(KVSS_EINVAL, "scale must be finite");
    if (kv->batch == 0) return ok();
    if (!q || !out || !tail_lo) return fail(KVSS_EINVAL, "q, out and tail_lo must be non-NULL");
    if (k_max > 0 && (!sel_idx || !sel_count))
        return fail(KVSS_EINVAL, "sel_idx and sel_count must be non-NULL when k_max > 0");
    const Plan p = draft_plan(kv, k_max, max_tail);
    const size_t need = partial_bytes((long)kv->batch * num_q_heads, p, kv->head_dim);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KVSS_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    static const int32_t* const kNoList = nullptr;
    kvss::AttnArgs a = attn_common(kv);
    a.q = q;
    a.Hq = num_q_heads;
    a.G = G;
    a.T = 1;
    a.R = G;
    a.sel_idx = k_max > 0 ? sel_idx : kNoList;
    a.sel_count = sel_count;
    a.tail_lo = tail_lo;
    a.k_max = k_max;
    if (k_max == 0) a.sel_count = tail_lo;   // read but clamped to k_max = 0
    a.scale_log2 = scale_log2(scale);
    a.out = out;
    a.lse = lse;
    return run_attention(a, p, true, kv->dtype, workspace, static_cast<hipStream_t>(stream));
}

int kvss_streaming_set(const int32_t* kv_lens, int batch, int num_kv_heads, int sink, int window,
                       int32_t* sel_idx, int32_t* sel_count, int32_t* tail_lo, void* stream) {
    if (batch < 0 || num_kv_heads <= 0 || sink < 0 || window < 0)
        return fail(KVSS_EINVAL, "batch, sink, window must be >= 0 and num_kv_heads >= 1");
    if (batch == 0) return ok();
    if (!kv_lens || !sel_count || !tail_lo || (sink > 0 && !sel_idx))
        return fail(KVSS_EINVAL, "kv_lens, sel_idx, sel_count and tail_lo must be non-NULL");
    return hip_status(kvss::launch_streaming_set(kv_lens, batch, num_kv_heads, sink, window, sel_idx,
                                                 sel_count, tail_lo, static_cast<hipStream_t>(stream)),
                      "streaming set launch");
}

size_t kvss_snapkv_workspace_bytes(const kvss_kv* kv, int num_q_heads, int w, int budget) {
    if (check_kv(kv) != KVSS_OK || num_q_heads <= 0 || num_q_heads % kv->num_kv_heads || w <= 0 ||
        budget <= w)
        return 0;
    return snap_layout(kv, num_q_heads, w, true).total;
}

int snapkv_select(const kvss_kv* kv, const void* q_obs, int num_q_heads, int w, int pool_kernel,
                  int budget, float scale, int32_t* sel_idx, int32_t* sel_count,
                  float* scores_out, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_kv(kv);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    if (w <= 0) return fail(KVSS_EINVAL, "observation window w must be >= 1");
    if (budget <= w) return fail(KVSS_EINVAL, "budget %d must exceed the window %d", budget, w);
    if (pool_kernel < 1 || pool_kernel % 2 == 0)
        return fail(KVSS_EINVAL, "pool_kernel %d must be odd and >= 1", pool_kernel);
    const int G = num_q_heads / kv->num_kv_heads;
    if (G * w > 256) return fail(KVSS_EUNSUPPORTED, "G * w = %d exceeds 256 rows per KV head", G * w);
    if (!isfinite(scale)) return fail(KVSS_EINVAL, "scale must be finite");
    if (kv->batch == 0) return ok();
    if (!q_obs || !sel_idx || !sel_count)
        return fail(KVSS_EINVAL, "q_obs, sel_idx and sel_count must be non-NULL");
    // The full requirement (workspace holds the scores too) is what the query reports; when the
    // caller keeps the scores, less is needed.
    const SnapLayout L = snap_layout(kv, num_q_heads, w, scores_out == nullptr);
    if (workspace_bytes < L.total || (L.total > 0 && !workspace))
        return fail(KVSS_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, L.total);
    char* ws = static_cast<char*>(workspace);
    kvss::SnapArgs a{};
    a.k = kv->k;
    a.block_table = kv->block_table;
    a.prompt_lens = kv->kv_lens;
    a.B = kv->batch;
    a.Hkv = kv->num_kv_heads;
    a.D = kv->head_dim;
    a.bs = kv->block_size;
    a.max_blocks = kv->max_blocks;
    a.num_blocks = kv->num_blocks;
    a.max_kv_len = kv->max_kv_len;
    a.dtype = kv->dtype;
    a.q_obs = q_obs;
    a.Hq = num_q_heads;
    a.G = G;
    a.w = w;
    a.R = G * w;
    a.scale_log2 = scale_log2(scale);
    a.nsplit1 = L.p1.nsplit;
    a.split_len1 = L.p1.split_len;
    a.part1 = reinterpret_cast<float*>(ws);
    a.rowc = reinterpret_cast<float*>(ws + L.part1);
    ws += L.part1 + L.rowc;
    a.scores = scores_out ? scores_out : reinterpret_cast<float*>(ws);
    a.n_stride = L.n_stride;
    a.pooled = reinterpret_cast<float*>(ws + L.scores);
    // (16-byte stores and loads; an unaligned workspace takes the path that re-reads K)
    a.xs = L.xs > 0 && aligned16(ws) ? reinterpret_cast<float*>(ws + L.scores + L.pooled) : nullptr;
    a.xs_stride = L.xs_stride;
    a.pool = pool_kernel;
    a.keep = budget - w;
    a.sel_idx = sel_idx;
    a.sel_count = sel_count;
    return hip_status(kvss::launch_snapkv(a, static_cast<hipStream_t>(stream)), "snapkv launch");
}

size_t kvss_accept_workspace_bytes(int batch, int gamma, int vocab) {
    if (batch < 0 || gamma < 0 || gamma > kMaxGamma || vocab <= 0) return 0;
    const kvss::AcceptPlan p = kvss::accept_plan(batch, gamma, vocab);
    return align_up(p.parts_bytes + p.bonus_bytes + p.race_bytes + p.dec_bytes);
}

int spec_accept(const float* target_logits, const float* draft_logits, const int32_t* draft_tokens,
                int batch, int gamma, int vocab, float temperature, uint64_t seed, uint64_t offset,
                int32_t* out_tokens, int32_t* out_num_accepted, float* row_stats, void* workspace,
                size_t workspace_bytes, void* stream) {
    if (batch < 0) return fail(KVSS_EINVAL, "batch must be >= 0");
    if (gamma < 0) return fail(KVSS_EINVAL, "gamma must be >= 0");
    if (gamma > kMaxGamma) return fail(KVSS_EUNSUPPORTED, "gamma %d exceeds %d", gamma, kMaxGamma);
    if (batch > kMaxGridYZ) return fail(KVSS_EUNSUPPORTED, "batch must be <= %d", kMaxGridYZ);
    if (vocab <= 0 || vocab >= (1 << 24)) return fail(KVSS_EINVAL, "vocab must be in [1, 2^24)");
    if (!temperature_ok(temperature))
        return fail(KVSS_EINVAL, "temperature must be finite and 0 or >= 1 / FLT_MAX");
    if (batch == 0) return ok();
    if (!target_logits || !out_tokens || !out_num_accepted || (gamma > 0 && !draft_tokens))
        return fail(KVSS_EINVAL, "target_logits, draft_tokens, out_tokens, out_num_accepted must be non-NULL");
    if (temperature > 0.f && gamma > 0 && !draft_logits)
        return fail(KVSS_EINVAL, "draft_logits must be non-NULL when temperature > 0");
    const size_t need = kvss_accept_workspace_bytes(batch, gamma, vocab);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KVSS_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    kvss::AcceptArgs a{};
    a.target = target_logits;
    a.draft = draft_logits;
    a.tokens = draft_tokens;
    a.B = batch;
    a.gamma = gamma;
    a.V = vocab;
    a.inv_temp = temperature > 0.f ? (float)(1.0 / (double)temperature) : 0.f;
    a.seed = seed;
    a.offset = offset;
    a.stats = row_stats;
    a.out_tokens = out_tokens;
    a.out_num = out_num_accepted;
    return hip_status(kvss::launch_accept(a, workspace, static_cast<hipStream_t>(stream)),
                      "accept launch");
}

size_t kvss_sample_workspace_bytes(int batch, int vocab) {
    if (batch < 0 || vocab <= 0) return 0;
    return align_up(kvss::sample_workspace_bytes(batch, vocab));
}

int draft_sample(const float* logits, int batch, int vocab, float temperature, uint64_t seed,
                 uint64_t offset, int step, int32_t* tokens, float* row_stats, void* workspace,
                 size_t workspace_bytes, void* stream) {
    if (batch < 0) return fail(KVSS_EINVAL, "batch must be >= 0");
    if (batch > kMaxGridYZ) return fail(KVSS_EUNSUPPORTED, "batch must be <= %d", kMaxGridYZ);
    if (vocab <= 0 || vocab >= (1 << 24)) return fail(KVSS_EINVAL, "vocab must be in [1, 2^24)");
    if (!temperature_ok(temperature))
        return fail(KVSS_EINVAL, "temperature must be finite and 0 or >= 1 / FLT_MAX");
    if (step < 0 || step > 0xffff) return fail(KVSS_EINVAL, "step must be in [0, 65535]");
    if (batch == 0) return ok();
    if (!logits || !tokens) return fail(KVSS_EINVAL, "logits and tokens must be non-NULL");
    const size_t need = kvss_sample_workspace_bytes(batch, vocab);
    if (workspace_bytes < need || !workspace)
        return fail(KVSS_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    kvss::SampleArgs a{};
    a.logits = logits;
    a.B = batch;
    a.V = vocab;
    a.inv_temp = temperature > 0.f ? (float)(1.0 / (double)temperature) : 0.f;
    a.seed = seed;
    a.offset = offset;
    a.stream_id = kDraftStream;
    a.step = step;
    a.tokens = tokens;
    a.stats = row_stats;
    return hip_status(kvss::launch_sample(a, workspace, static_cast<hipStream_t>(stream)),
                      "draft sample launch");
}

int kvss_kv_append(const kvss_kv* kv, const void* k_new, const void* v_new, int T,
                   const int32_t* start, void* stream) {
    int rc = check_kv(kv);
    if (rc) return rc;
    if (T < 0) return fail(KVSS_EINVAL, "T must be >= 0 (got %d)", T);
    if (kv->batch == 0 || T == 0) return ok();
    if ((long long)kv->batch * T > 0x7fffffffLL)
        return fail(KVSS_EUNSUPPORTED, "batch * T = %lld rows exceeds 2^31 - 1", (long long)kv->batch * T);
    if (!k_new || !v_new || !start) return fail(KVSS_EINVAL, "k_new, v_new and start must be non-NULL");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kv->k) || !aligned16(kv->v))
        return fail(KVSS_EINVAL, "k, v, k_new and v_new must be 16-byte aligned");
    kvss::AppendArgs a{};
    a.k = const_cast<void*>(kv->k);
    a.v = const_cast<void*>(kv->v);
    a.block_table = kv->block_table;
    a.B = kv->batch;
    a.Hkv = kv->num_kv_heads;
    a.bs = kv->block_size;
    a.max_blocks = kv->max_blocks;
    a.num_blocks = kv->num_blocks;
    a.row_bytes = kv->head_dim * (kv->dtype == KVSS_BF16 ? 2 : 4);
    a.k_new = k_new;
    a.v_new = v_new;
    a.T = T;
    a.start = start;
    return hip_status(kvss::launch_kv_append(a, static_cast<hipStream_t>(stream)), "kv append launch");
}

int kvss_draft_cache_build(const kvss_kv* src, const int32_t* sel_idx, const int32_t* sel_count,
                           int k_max, const int32_t* tail_lo, int max_tail, const kvss_kv* dst,
                           int32_t* dst_lens, void* stream) {
    int rc = check_kv(src);
    if (rc) return rc;
    if ((rc = check_kv(dst))) return rc;
    if (k_max < 0 || max_tail < 0)
        return fail(KVSS_EINVAL, "k_max (%d) and max_tail (%d) must be >= 0", k_max, max_tail);
    if (dst->batch != src->batch || dst->num_kv_heads != src->num_kv_heads ||
        dst->head_dim != src->head_dim || dst->dtype != src->dtype)
        return fail(KVSS_EINVAL, "dst must match src in batch, num_kv_heads, head_dim and dtype");
    if (src->batch == 0) return ok();
    if ((long long)k_max + max_tail > (long long)dst->max_blocks * dst->block_size)
        return fail(KVSS_EINVAL, "k_max + max_tail = %lld exceeds the compact capacity %lld",
                    (long long)k_max + max_tail, (long long)dst->max_blocks * dst->block_size);
    if (k_max > 0 && (!sel_idx || !sel_count))
        return fail(KVSS_EINVAL, "sel_idx and sel_count must be non-NULL when k_max > 0");
    if (!tail_lo || !dst_lens) return fail(KVSS_EINVAL, "tail_lo and dst_lens must be non-NULL");
    if (!aligned16(src->k) || !aligned16(src->v) || !aligned16(dst->k) || !aligned16(dst->v))
        return fail(KVSS_EINVAL, "cache tensors must be 16-byte aligned");
    if (src->k == dst->k || src->v == dst->v || src->k == dst->v || src->v == dst->k)
        return fail(KVSS_EINVAL, "dst must not alias src");
    kvss::CompactArgs a{};
    a.k = src->k;
    a.v = src->v;
    a.block_table = src->block_table;
    a.kv_lens = src->kv_lens;
    a.B = src->batch;
    a.Hkv = src->num_kv_heads;
    a.bs = src->block_size;
    a.max_blocks = src->max_blocks;
    a.num_blocks = src->num_blocks;
    a.max_kv_len = src->max_kv_len;
    a.row_bytes = src->head_dim * (src->dtype == KVSS_BF16 ? 2 : 4);
    a.dtype = src->dtype;
    a.sel_idx = k_max > 0 ? sel_idx : nullptr;
    a.sel_count = k_max > 0 ? sel_count : nullptr;
    a.tail_lo = tail_lo;
    a.k_max = k_max;
    a.max_tail = max_tail;
    a.dst_k = const_cast<void*>(dst->k);
    a.dst_v = const_cast<void*>(dst->v);
    a.dst_table = dst->block_table;
    a.dst_bs = dst->block_size;
    a.dst_max_blocks = dst->max_blocks;
    a.dst_num_blocks = dst->num_blocks;
    a.dst_lens = dst_lens;
    return hip_status(kvss::launch_compact_build(a, static_cast<hipStream_t>(stream)),
                      "draft cache build launch");
}

// Dynamic Top-K draft: SnapKV-rule selection with the draft query as a one-token window,
// then the gathered draft. Workspace = selection scratch | sel | count | tail_lo | draft.
struct TopkLayout {
    size_t snap, sel, cnt, tail, draft, total;
};

static TopkLayout topk_layout(const kvss_kv* kv, int num_q_heads, int k) {
    TopkLayout t{};
    t.snap = align_up(snap_layout(kv, num_q_heads, 1, true).total);
    t.sel = align_up((size_t)kv->batch * kv->num_kv_heads * k * sizeof(int32_t));
    t.cnt = align_up((size_t)kv->batch * sizeof(int32_t));
    t.tail = t.cnt;
    t.draft = align_up(partial_bytes((long)kv->batch * num_q_heads, draft_plan(kv, k, 1), kv->head_dim));
    t.total = t.snap + t.sel + t.cnt + t.tail + t.draft;
    return t;
}

size_t kvss_topk_workspace_bytes(const kvss_kv* kv, int num_q_heads, int k) {
    if (check_kv(kv) != KVSS_OK || num_q_heads <= 0 || num_q_heads % kv->num_kv_heads || k <= 0)
        return 0;
    return topk_layout(kv, num_q_heads, k).total;
}

int draft_attn_topk(const kvss_kv* kv, const void* q, int num_q_heads, int k, float scale,
                    float* out, float* lse, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int rc = check_kv(kv);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads))) return rc;
    const int G = num_q_heads / kv->num_kv_heads;
    if (G > 32) return fail(KVSS_EUNSUPPORTED, "G = %d exceeds 32 query rows per KV head", G);
    if (k <= 0) return fail(KVSS_EINVAL, "k must be >= 1 (got %d)", k);
    if (!isfinite(scale)) return fail(KVSS_EINVAL, "scale must be finite");
    if (kv->batch == 0) return ok();
    if (!q || !out) return fail(KVSS_EINVAL, "q and out must be non-NULL");
    const TopkLayout t = topk_layout(kv, num_q_heads, k);
    if (workspace_bytes < t.total || !workspace)
        return fail(KVSS_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, t.total);
    char* ws = static_cast<char*>(workspace);
    int32_t* sel = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(ws + t.snap);
    int32_t* cnt = sel_count ? sel_count : reinterpret_cast<int32_t*>(ws + t.snap + t.sel);
    int32_t* tail = reinterpret_cast<int32_t*>(ws + t.snap + t.sel + t.cnt);
    // The draft query [B, Hq, D] is the one-token observation window [B, Hq, 1, D].
    if ((rc = snapkv_select(kv, q, num_q_heads, 1, 1, k + 1, scale, sel, cnt, nullptr, ws, t.snap,
                            stream)))
        return rc;
    hipError_t e = kvss::launch_tail_lo(kv->kv_lens, kv->batch, kv->max_kv_len, 1, tail,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e, "tail launch");
    return draft_attn_sparse(kv, q, num_q_heads, sel, cnt, k, tail, 1, scale, out, lse,
                             ws + t.snap + t.sel + t.cnt + t.tail, t.draft, stream);
}

int kvss_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (bytes == 0) return ok();
    if (!src || !sink) return fail(KVSS_EINVAL, "src and sink must be non-NULL");
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return fail(KVSS_EINVAL, "src must be 16-byte aligned");
    return hip_status(kvss::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)),
                      "stream read launch");
}

int kvss_philox4x32_10(const uint32_t* counters, int64_t n, uint64_t seed, uint32_t* out,
                       void* stream) {
    if (n < 0) return fail(KVSS_EINVAL, "n must be >= 0 (got %lld)", (long long)n);
    if (n == 0) return ok();
    if (!counters || !out) return fail(KVSS_EINVAL, "counters and out must be non-NULL");
    if (!aligned16(counters) || !aligned16(out))
        return fail(KVSS_EINVAL, "counters and out must be 16-byte aligned");
    if (n > ((int64_t)1 << 31))      // one thread per counter: the grid stays below 2^32 threads
        return fail(KVSS_EUNSUPPORTED, "n = %lld exceeds 2^31 counters", (long long)n);
    return hip_status(kvss::launch_philox(counters, n, seed, out, static_cast<hipStream_t>(stream)),
                      "philox launch");
}

}  // extern "C"
