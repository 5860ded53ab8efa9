// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvss {

// Physical-row entries one bf16 attention workgroup keeps in LDS: per key for a gathered set,
// per cache block for a dense range.
constexpr int kMfmaTableEntries = 4096;

// Candidate keys one workgroup of the bf16 SnapKV column-score pass covers.
constexpr int kSnapColKeys = 4096;
constexpr int kSnapTableEntries = 1024;     // block bases per SnapKV row-statistics split

// One attention launch: R = G * T query rows per (sequence, KV head) over a key set that is
// either the dense causal range [0, L) (verify) or a gathered list + dense tail (draft).
struct AttnArgs {
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* kv_lens;
    int B, Hkv, D, bs, max_blocks, num_blocks, max_kv_len;
    const void* q;              // [B, Hq, T, D]
    int Hq, G, T, R;
    const int32_t* sel_idx;     // gather mode only: [B, Hkv, k_max]
    const int32_t* sel_count;   // [B]
    const int32_t* tail_lo;     // [B]
    int k_max;
    float scale_log2;           // softmax scale * log2(e)
    int nsplit, split_len;      // virtual key range of split s: [s*split_len, (s+1)*split_len)
    float* out;                 // [B, Hq, T, D]
    float* lse;                 // [B, Hq, T] or null
    float* part;                // [B*Hq*T, nsplit, D + 2] when nsplit > 1
};

hipError_t launch_attn_mfma(const AttnArgs& a, bool gather, hipStream_t s);
hipError_t launch_attn_simple(const AttnArgs& a, bool gather, hipStream_t s);
hipError_t launch_merge(const float* part, int rows, int nsplit, int D, float* out, float* lse,
                        hipStream_t s);

struct SnapArgs {
    const void* k;
    const int32_t* block_table;
    const int32_t* prompt_lens;
    int B, Hkv, D, bs, max_blocks, num_blocks, max_kv_len, dtype;
    const void* q_obs;          // [B, Hq, w, D]
    int Hq, G, w, R;            // R = G * w rows per (sequence, KV head)
    float scale_log2;
    int nsplit1, split_len1;    // pass-1 key splits
    float* part1;               // [B*Hkv*R, nsplit1, 2] row (max, sum) partials, log2 domain
    float* rowc;                // [B*Hkv*R] -(max + log2 sum) per row, merged from part1
    float* scores;              // [B, Hkv, n_stride] column scores
    int n_stride;               // max_kv_len - w
    float* pooled;              // [B, Hkv, n_stride] workspace
    float* xs;                  // [B, Hkv, R, xs_stride] scaled candidate scores, or null
    int xs_stride;              // n_stride rounded up to a multiple of 4
    int pool, keep;             // pool kernel, kept count budget - w
    int32_t* sel_idx;           // [B, Hkv, keep]
    int32_t* sel_count;         // [B]
};

hipError_t launch_snapkv(const SnapArgs& a, hipStream_t s);
hipError_t launch_snapkv_mfma_passes(const SnapArgs& a, hipStream_t s);

// Append T rows per sequence to a paged cache (k_new / v_new [B, Hkv, T, D]).
struct AppendArgs {
    void* k;
    void* v;
    const int32_t* block_table;
    int B, Hkv, bs, max_blocks, num_blocks, row_bytes;
    const void* k_new;
    const void* v_new;
    int T;
    const int32_t* start;       // [B] logical position of row 0
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);

// Copy each (sequence, KV head)'s draft set (listed rows, then the tail) into a compact cache.
struct CompactArgs {
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* kv_lens;
    int B, Hkv, bs, max_blocks, num_blocks, max_kv_len, row_bytes, dtype;
    const int32_t* sel_idx;     // [B, Hkv, k_max] or null when k_max == 0
    const int32_t* sel_count;   // [B] or null when k_max == 0
    const int32_t* tail_lo;     // [B]
    int k_max, max_tail;
    void* dst_k;
    void* dst_v;
    const int32_t* dst_table;   // [B, dst_max_blocks]
    int dst_bs, dst_max_blocks, dst_num_blocks;
    int32_t* dst_lens;          // [B]
};

hipError_t launch_compact_build(const CompactArgs& a, hipStream_t s);

hipError_t launch_tail_lo(const int32_t* kv_lens, int B, int max_kv_len, int back, int32_t* tail_lo,
                          hipStream_t s);

hipError_t launch_streaming_set(const int32_t* kv_lens, int B, int Hkv, int sink, int window,
                                int32_t* sel_idx, int32_t* sel_count, int32_t* tail_lo,
                                hipStream_t s);

struct AcceptArgs {
    const float* target;        // [B, gamma+1, V]
    const float* draft;         // [B, gamma, V]
    const int32_t* tokens;      // [B, gamma]
    int B, gamma, V;
    float inv_temp;             // 0 => greedy
    uint64_t seed, offset;
    float* stats;               // [B, 2*gamma+1, 4] or null
    int32_t* out_tokens;        // [B, gamma+1]
    int32_t* out_num;           // [B]
};

// Workspace carve-up of one acceptance call: per-row slice partials, the statistics pass's race
// keys over p_gamma, the race keys per slice, the decision per sequence.
struct AcceptPlan {
    int nslice, nrace;
    size_t parts_bytes, bonus_bytes, race_bytes, dec_bytes;
};
AcceptPlan accept_plan(int B, int gamma, int V);
hipError_t launch_accept(const AcceptArgs& a, void* workspace, hipStream_t s);

// Draft-token sampler: one logit row per sequence, one pass (slice kernel + finalize).
struct SampleArgs {
    const float* logits;        // [B, V]
    int B, V;
    float inv_temp;             // 0 => greedy
    uint64_t seed, offset;
    int stream_id, step;        // Philox stream and position of the race
    int32_t* tokens;            // [B]
    float* stats;               // [B, 4] or null
};
int sample_slices(int V);
size_t sample_workspace_bytes(int B, int V);
hipError_t launch_sample(const SampleArgs& a, void* workspace, hipStream_t s);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_philox(const uint32_t* counters, int64_t n, uint64_t seed, uint32_t* out,
                         hipStream_t s);

}  // namespace kvss
