/*
 * kvss.h -- C ABI of libkvss: the KV-cache hot path of sparse-KV self-speculative decoding
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations follow "MagicDec: Breaking the Latency-Throughput Tradeoff for Long Context
 * Generation with Speculative Decoding" (arXiv 2408.11049v5). Its cost model names the three
 * timed steps of one speculative round -- KV selection T_select(B,S,K) and sparse draft
 * decoding T_D(B,K) (Section 4.1, Eq. (3)), verification of gamma tokens T_V(B,S,gamma)
 * (Section 3.1, Eq. (2)) -- and the accepted-token count Omega(gamma, alpha) (Section 3.1,
 * Eq. (1)). Each maps to one call below:
 *
 *   snapkv_select      T_select : static SnapKV selection at prefill (Section 4.4, App. A.1)
 *   kvss_streaming_set T_select : StreamingLLM sink + window set (Section 5.1, Table 1)
 *   draft_attn_sparse  T_D      : one draft query per sequence over a sparse subset
 *   draft_attn_topk    T_select + T_D : the dynamic Top-K draft, subset searched every step
 *   verify_attn_full   T_V      : gamma + 1 causal queries per sequence over the full cache
 *   spec_accept        Omega    : greedy / rejection-sampling acceptance
 *   draft_sample       the draft token of each draft step (greedy or sampled)
 * and the cache maintenance around them (Section 3.1; Appendix A.1, Fig. 8):
 *   kvss_kv_append          append the newly scored tokens' K/V rows to a paged cache
 *   kvss_draft_cache_build  materialise the compressed draft cache once at prefill
 * plus kvss_philox4x32_10 (the generator behind every sampled draw, to replay one) and
 * kvss_stream_read (a plain read, the bandwidth reference the kernels are measured against).
 *
 * Conventions (all calls)
 *   - Every pointer argument that names a tensor is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains device memory (the one exception is the fixed
 *     per-GPU scratch array of verify_attn_full_noalloc, part of the loaded code object).
 *     Scratch space comes from the caller's `workspace` buffer, whose required size the
 *     matching *_workspace_bytes query returns for the same shape arguments (0 is a valid
 *     size; workspace may then be NULL).
 *     A workspace must not be shared by calls that may run concurrently.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls enqueue
 *     kernels and return without synchronising; outputs are valid once the stream has
 *     reached the enqueued work.
 *   - Return value: KVSS_OK (0) or a negative KVSS_E* code. All argument checks run on the
 *     host before any HIP call; on error nothing is enqueued and kvss_last_error() returns a
 *     thread-local message. No C++ exception crosses this boundary.
 *   - Results are bitwise deterministic for fixed inputs and shapes (no floating-point
 *     atomics, fixed split plans).
 *   - Tensors are dense, row-major, in the shapes given; strides are not accepted.
 */
#ifndef KVSS_H
#define KVSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define KVSS_API __attribute__((visibility("default")))
#else
#define KVSS_API
#endif

/* Status codes. */
#define KVSS_OK 0
#define KVSS_EINVAL (-1)        /* bad shape, pointer, length or budget                     */
#define KVSS_EUNSUPPORTED (-2)  /* dtype, head_dim, block size or row count not compiled     */
#define KVSS_EWORKSPACE (-3)    /* workspace smaller than the *_workspace_bytes query        */
#define KVSS_EHIP (-4)          /* a HIP launch failed; the message carries the HIP string   */

/* Storage types of K, V and queries. Attention outputs are always float32. */
#define KVSS_F32 0
#define KVSS_BF16 1

/*
 * Paged KV cache of one layer (MagicDec Sections 1 and 3.2: the per-layer KV cache is the
 * dominant bandwidth term; the paper fixes no layout, this library uses paged blocks).
 *   k, v        [num_blocks, num_kv_heads, block_size, head_dim] of `dtype`
 *   block_table int32 [batch, max_blocks]: logical row j of sequence b is physical block
 *               block_table[b, j / block_size], offset j % block_size. Entries past a
 *               sequence's last block are never read.
 *   kv_lens     int32 [batch] (device): rows cached per sequence.
 *   max_kv_len  host-side upper bound of kv_lens, used to size launches; it must satisfy
 *               max_kv_len <= max_blocks * block_size. Kernels clamp kv_lens[b] to it.
 * Kernels that meet a block id outside [0, num_blocks) write NaN to the outputs of the
 * affected sequence instead of reading out of bounds.
 * Supported: dtype KVSS_BF16 or KVSS_F32; head_dim 64 or 128; block_size a multiple of 16.
 */
typedef struct kvss_kv {
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* kv_lens;
    int32_t batch;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t max_kv_len;
    int32_t dtype;
} kvss_kv;

/* Thread-local description of the last error (empty string after success). */
KVSS_API const char* kvss_last_error(void);

/* Library ABI version (increments on any signature or semantic change). */
KVSS_API int kvss_version(void);

/*
 * verify_attn_full -- T = gamma + 1 causal queries per sequence over the full cache.
 * MagicDec Section 3.1 (T_V(B,S,gamma), Eq. (2)) and Section 3.2: verification reads the same
 * KV cache as plain decoding, which is what makes it cheap in the long-context regime.
 *   q    [batch, num_q_heads, T, head_dim] of kv->dtype. Query t of sequence b sits at
 *        position kv_lens[b] - T + t (the T new rows are already in the cache) and attends to
 *        rows [0, kv_lens[b] - T + t]; q-head h reads KV head h / G, G = num_q_heads /
 *        num_kv_heads. A query with an empty range yields out = 0, lse = -inf.
 *   out  float32 [batch, num_q_heads, T, head_dim]: softmax(scale * q K^T) V.
 *   lse  float32 [batch, num_q_heads, T] or NULL: natural-log sum of exp(scale * q k).
 * Limits: G * T <= 32.
 */
KVSS_API size_t kvss_verify_workspace_bytes(const kvss_kv* kv, int num_q_heads, int T);
KVSS_API int verify_attn_full(const kvss_kv* kv, const void* q, int num_q_heads, int T, float scale,
                     float* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * verify_attn_full_noalloc -- verify_attn_full for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It
 * computes exactly what verify_attn_full computes, with the same kernels and split plan, so
 * the results are bit-identical; the split partials live in a device array the library owns
 * instead of a caller workspace.
 *   Arguments as for verify_attn_full, without the workspace.
 *   Scratch limit: 32 MiB (33554432 bytes). A shape whose kvss_verify_workspace_bytes exceeds
 *   it returns KVSS_EWORKSPACE and enqueues nothing; every shape with a workspace need of 0
 *   (an unsplit plan) is accepted.
 *   The array is one per GPU, holds its 32 MiB until the process ends, and keeps the last
 *   call's contents (nothing in it needs to start at zero). The first call on a device looks
 *   its address up (hipGetSymbolAddress), preferably outside graph capture. Calls that may
 *   overlap on one GPU (other streams, other threads) race on the array: serialise them.
 *   No hipMalloc, hipFree or allocating library routine is called.
 */
KVSS_API int verify_attn_full_noalloc(const kvss_kv* kv, const void* q, int num_q_heads, int T,
                                      float scale, float* out, float* lse, void* stream);

/*
 * draft_attn_sparse -- one draft query per sequence over a sparse subset of the cache.
 * MagicDec Section 4.1, Eq. (3) (T_D(B,K): decoding against K selected rows) and Appendix A.1,
 * Fig. 8 (self-speculation drafts from a compressed view of the target's own cache).
 *   q         [batch, num_q_heads, head_dim] of kv->dtype.
 *   sel_idx   int32 [batch, num_kv_heads, k_max]: selected positions, ascending, each in
 *             [0, tail_lo[b]); entries i >= sel_count[b] are ignored. Entries outside
 *             [0, min(tail_lo[b], kv_lens[b])) are skipped. May be NULL when k_max == 0.
 *   sel_count int32 [batch] (may be NULL when k_max == 0).
 *   tail_lo   int32 [batch]: the dense tail [tail_lo[b], kv_lens[b]) is attended as well.
 *   max_tail  host-side estimate of max_b (kv_lens[b] - tail_lo[b]); it only shapes the launch
 *             (the whole set is attended whatever the actual tail length).
 *   out       float32 [batch, num_q_heads, head_dim]; lse float32 [batch, num_q_heads] or NULL.
 * Limits: G <= 32, k_max >= 0, max_tail >= 0.
 */
KVSS_API size_t kvss_draft_workspace_bytes(const kvss_kv* kv, int num_q_heads, int k_max, int max_tail);
KVSS_API int draft_attn_sparse(const kvss_kv* kv, const void* q, int num_q_heads,
                      const int32_t* sel_idx, const int32_t* sel_count, int k_max,
                      const int32_t* tail_lo, int max_tail, float scale, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvss_streaming_set -- StreamingLLM draft set in the draft_attn_sparse encoding.
 * MagicDec Section 5.1 (StreamingLLM-style sparse KV drafting) and Table 1 (budget 512).
 * For L = kv_lens[b]: sel_idx[b, g, j] = j for j < min(sink, L), else -1 (j < sink);
 * sel_count[b] = min(sink, L); tail_lo[b] = max(sink, L - window). The attended set is the
 * first `sink` rows plus the last `window` rows (the current token included).
 *   sel_idx int32 [batch, num_kv_heads, sink]; sel_count, tail_lo int32 [batch].
 */
KVSS_API int kvss_streaming_set(const int32_t* kv_lens, int batch, int num_kv_heads, int sink,
                       int window, int32_t* sel_idx, int32_t* sel_count, int32_t* tail_lo,
                       void* stream);

/*
 * snapkv_select -- static SnapKV selection of the draft cache from the prompt.
 * MagicDec Section 4.4 (static selection: no per-query search cost), Section 5.2 (SnapKV
 * budgets) and Appendix A.1 (built during prefill). For sequence b with P = kv_lens[b] prompt
 * rows, q-head h of group g and observation query i < w at position P - w + i:
 *   1. softmax of scale * q k over keys [0, P - w + i];
 *   2. c[b, g, j] = sum over h in g, i < w of those probabilities, j in [0, P - w);
 *   3. pooled = centred max-pool of width pool_kernel (odd) over [0, P - w);
 *   4. keep the k = budget - w largest pooled values (ties: lower position), ascending.
 *   q_obs      [batch, num_q_heads, w, head_dim] of kv->dtype.
 *   sel_idx    int32 [batch, num_kv_heads, budget - w], -1 padded.
 *   sel_count  int32 [batch] = min(budget - w, max(P - w, 0)).
 *   scores_out float32 [batch, num_kv_heads, max_kv_len - w] or NULL: the column scores c
 *              (entries j >= P - w of a shorter prompt are left untouched).
 * The draft then attends sel_idx plus the dense tail [P - w, L).
 * Limits: 0 < w < budget, G * w <= 256, pool_kernel odd and >= 1.
 * Workspace: kvss_snapkv_workspace_bytes. With bf16 and R = G * w <= 16 rows (4 R < head_dim)
 * it includes the first pass's scaled scores, R floats per candidate, which the second pass
 * reads instead of K; a workspace that is not 16-byte aligned makes the second pass re-read K
 * (same selection, scores equal to float32 rounding).
 */
KVSS_API size_t kvss_snapkv_workspace_bytes(const kvss_kv* kv, int num_q_heads, int w, int budget);
KVSS_API int snapkv_select(const kvss_kv* kv, const void* q_obs, int num_q_heads, int w, int pool_kernel,
                  int budget, float scale, int32_t* sel_idx, int32_t* sel_count,
                  float* scores_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_accept -- acceptance of gamma draft tokens against gamma + 1 target positions.
 * MagicDec Section 3.1 (speculative decoding of Leviathan et al.; Eq. (1) gives the expected
 * number of emitted tokens) and Section 5.1 (greedy decoding in all end-to-end runs).
 *   target_logits float32 [batch, gamma + 1, vocab]; draft_logits float32 [batch, gamma,
 *   vocab] (not read when temperature == 0; may then be NULL); draft_tokens int32
 *   [batch, gamma], each in [0, vocab).
 *   temperature == 0: greedy. Draft token i is accepted while it equals the target argmax at
 *     position i (ties: lowest id); the first mismatch emits the target argmax there; if all
 *     match, the argmax at position gamma is appended. The argmax is taken over a row's non-NaN
 *     logits; a row with none has argmax -1, which then is the emitted token.
 *   temperature > 0: rejection sampling with p = softmax(target / temperature), q = softmax(
 *     draft / temperature). Position i accepts when u_i < p_i(x_i) / q_i(x_i); the first
 *     rejection emits a draw from max(0, p_i - q_i) (from p_i if that is all zero); if all are
 *     accepted a draw from p_gamma is appended. Draws are exponential races,
 *     argmin_x -log(u'_x) / w(x). Uniforms come from Philox4x32-10 (Salmon et al., SC'11) with
 *     key (seed low, seed high) and counter (block j, stream << 16 | position, b,
 *     offset low 32 bits); stream 0 word 0 gives u_i, stream 1 word x % 4 of block x / 4
 *     gives u'_x; a 32-bit word x maps to (x >> 9) * 2^-23 + 2^-24. Callers advance `offset`
 *     between calls that share a seed.
 *   Rows holding NaN or no finite logit give unspecified sampling draws (never an error).
 *   The workspace holds the call's partials (no clearing needed); calls that overlap in time
 *   need separate workspaces.
 *   Limits: 0 <= gamma <= 31 and batch <= 65535 (KVSS_EUNSUPPORTED above), 1 <= vocab < 2^24.
 *   out_tokens       int32 [batch, gamma + 1]: emitted tokens, then -1.
 *   out_num_accepted int32 [batch]: accepted draft tokens, 0 .. gamma.
 *   row_stats        float32 [batch, 2 * gamma + 1, 4] or NULL: per logit row (target rows
 *                    0..gamma, then draft rows 0..gamma-1) the max of z / temperature, the sum
 *                    of exp(z / temperature - max), z / temperature at the row's draft token
 *                    (0 for the last target row), and the argmax as a float (-1 for a row
 *                    with no non-NaN logit). With
 *                    temperature == 0 only the argmax of target rows is filled; every other
 *                    entry, the draft rows included, is written as 0.
 */
KVSS_API size_t kvss_accept_workspace_bytes(int batch, int gamma, int vocab);
KVSS_API int spec_accept(const float* target_logits, const float* draft_logits,
                const int32_t* draft_tokens, int batch, int gamma, int vocab, float temperature,
                uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_num_accepted,
                float* row_stats, void* workspace, size_t workspace_bytes, void* stream);

/*
 * draft_attn_topk -- dynamic Top-K draft attention (MagicDec Fig. 1(c): TopK attention has
 * the highest acceptance of the drafts compared; Section 4.4, Static vs Dynamic: its subset is
 * searched anew for every draft query, so the selection cost T_select(B, S, K) is paid on every
 * draft step). One draft query per sequence (position kv_lens[b] - 1) attends to itself and to
 * the k keys of [0, kv_lens[b] - 1) with the largest sum, over the G query heads of its KV head,
 * of their softmax probabilities (for G = 1: the k largest raw scores); ties go to the lower
 * position. This is snapkv_select with the query as a one-token window (w = 1, pool = 1,
 * budget = k + 1) followed by draft_attn_sparse over that list and the tail [L - 1, L);
 * both read the whole cache prefix, which is the dynamic selection's cost.
 *   q         [batch, num_q_heads, head_dim] of kv->dtype
 *   k         keys kept per (sequence, KV head), >= 1; sequences with fewer candidates keep all
 *   out, lse  as for draft_attn_sparse (lse nullable)
 *   sel_idx   nullable int32 [batch, num_kv_heads, k]: the kept positions, ascending, -1 pad
 *   sel_count nullable int32 [batch]: kept count min(k, L - 1)
 * Workspace: kvss_topk_workspace_bytes(kv, num_q_heads, k). Supported: G <= 32.
 */
KVSS_API size_t kvss_topk_workspace_bytes(const kvss_kv* kv, int num_q_heads, int k);
KVSS_API int draft_attn_topk(const kvss_kv* kv, const void* q, int num_q_heads, int k, float scale,
                             float* out, float* lse, int32_t* sel_idx, int32_t* sel_count,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * draft_sample -- the draft token of one draft step (MagicDec Section 3.1: the draft proposes
 * the gamma tokens the target verifies; Section 5.1 drafts greedily). From the draft's logits
 * [batch, vocab] (fp32): temperature 0 takes the argmax over the non-NaN logits (ties to the
 * lowest id; -1 for a row with none); temperature
 * t > 0 draws from softmax(logits / t) by the exponential race spec_accept uses, on a Philox
 * stream of its own (stream 2, position `step`, same key and offset conventions), so the draft
 * token and the later acceptance draws are independent. The normaliser of softmax is common to
 * every token, so the race winner is argmin_x (ln E_x - z_x / t) and each row is read once.
 *   step       draft step index within the round, in [0, 65535]
 *   tokens     int32 [batch] (device), written
 *   row_stats  nullable float [batch, 4]: max of z / t, sum of exp(z / t - max), 0, argmax
 *              (at temperature 0 only the argmax is meaningful: the first two are 0)
 * Workspace: kvss_sample_workspace_bytes(batch, vocab). vocab < 2^24; batch <= 65535
 * (KVSS_EUNSUPPORTED above).
 */
KVSS_API size_t kvss_sample_workspace_bytes(int batch, int vocab);
KVSS_API int draft_sample(const float* logits, int batch, int vocab, float temperature,
                          uint64_t seed, uint64_t offset, int step, int32_t* tokens,
                          float* row_stats, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * kvss_kv_append -- write T new K/V rows per sequence into a paged cache (MagicDec
 * Section 3.1: the gamma + 1 tokens a verify pass scores are part of the cache it attends
 * to; Appendix A.1, Fig. 8: the compressed draft cache grows the same way).
 *   kv            the cache written; the call writes through kv->k and kv->v (kv_lens and
 *                 max_kv_len are not used: the caller advances its lengths itself)
 *   k_new, v_new  [batch, num_kv_heads, T, head_dim] of kv->dtype, 16-byte aligned
 *   start         int32 [batch] (device): row t of sequence b goes to logical position
 *                 start[b] + t, i.e. physical block block_table[b, pos / block_size] at
 *                 offset pos % block_size.
 * A row whose position is negative or >= max_blocks * block_size, or whose block id lies
 * outside [0, num_blocks), is not written. Sequences must not share the blocks being
 * written (concurrent writes to one row are not ordered). T == 0 or batch == 0: no-op.
 */
KVSS_API int kvss_kv_append(const kvss_kv* kv, const void* k_new, const void* v_new, int T,
                            const int32_t* start, void* stream);

/*
 * kvss_draft_cache_build -- materialise the compressed draft cache once at prefill (MagicDec
 * Appendix A.1, Fig. 8: the static compressed KV is built once at prefill and then read for
 * drafting). For every (sequence b, KV head g) the compact cache `dst` receives, as logical
 * rows 0 .. n_b - 1:
 *     src rows sel_idx[b, g, 0 : n] (n = sel_count[b] clamped to [0, k_max]), in list order,
 *     then src rows [tail_lo[b], L_b), L_b = src->kv_lens[b] clamped to src->max_kv_len,
 * and dst_lens[b] = n_b. A plain decode over dst (verify_attn_full with T = 1, kv_lens =
 * dst_lens) then attends to exactly the set draft_attn_sparse reads from src.
 *   src           the target cache (read only)
 *   sel_idx       int32 [batch, num_kv_heads, k_max], ascending positions < tail_lo[b]
 *                 (as snapkv_select or kvss_streaming_set produce); NULL allowed if k_max == 0
 *   sel_count     int32 [batch]; NULL allowed if k_max == 0
 *   tail_lo       int32 [batch]
 *   max_tail      host bound on L_b - tail_lo[b]
 *   dst           compact cache, same batch, num_kv_heads, head_dim and dtype as src, its own
 *                 block table and storage (must not alias src); k_max + max_tail must not
 *                 exceed dst->max_blocks * dst->block_size. dst->kv_lens and max_kv_len are
 *                 not used.
 *   dst_lens      int32 [batch] (device), written.
 * A compact cache holds one row per slot, so inputs it cannot represent are made visible
 * rather than dropped: a listed position outside [0, tail_lo[b]) or a src block id outside
 * [0, src->num_blocks) gives a row of NaN, and a sequence whose tail exceeds max_tail gets
 * NaN in every slot (its length is then n + max_tail). A dst block id outside
 * [0, dst->num_blocks) is not written.
 */
KVSS_API int kvss_draft_cache_build(const kvss_kv* src, const int32_t* sel_idx,
                                    const int32_t* sel_count, int k_max, const int32_t* tail_lo,
                                    int max_tail, const kvss_kv* dst, int32_t* dst_lens,
                                    void* stream);

/*
 * kvss_stream_read -- measurement reference, not part of the method: reads `bytes` (rounded
 * down to a multiple of 16) of the device buffer `src` (16-byte aligned) with 16-byte loads, the
 * practical HBM read ceiling against which the attention kernels' bandwidth is also reported.
 * `sink` is a device uint32 that is written only in a data-dependent corner case.
 */
KVSS_API int kvss_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * kvss_philox4x32_10 -- the generator behind the draws of spec_accept and draft_sample,
 * evaluated on caller-given counters (MagicDec Section 3.1: speculative sampling consumes
 * uniform draws; the paper leaves their source open, and this library takes Philox4x32-10 of
 * Salmon et al., SC'11, with the counter layouts documented above). A caller can replay any
 * draw the library made, e.g. u_i of spec_accept is word 0 of counter (0, i, b, offset low
 * 32 bits) under seed `seed`.
 *   counters  uint32 [n, 4] (device, 16-byte aligned): counter words (c0, c1, c2, c3)
 *   seed      the key is (seed low 32 bits, seed high 32 bits)
 *   out       uint32 [n, 4] (device, 16-byte aligned), written: the four output words
 * n == 0 is a no-op; n < 0 or a NULL / misaligned pointer is KVSS_EINVAL; n > 2^31 is
 * KVSS_EUNSUPPORTED.
 */
KVSS_API int kvss_philox4x32_10(const uint32_t* counters, int64_t n, uint64_t seed, uint32_t* out,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSS_H */
