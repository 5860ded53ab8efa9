// bf16 split-KV attention on gfx950 matrix cores: verify (gamma + 1 causal queries per
// sequence over the full cache) and sparse draft (one query over a gathered subset).
//
// MagicDec (arXiv 2408.11049v5) Section 3.2 explains why this is the hot path: in the
// long-context, large-batch regime the per-step KV load dominates, and verification costs
// about one decode because both stream the same cache. The kernel therefore streams each
// (sequence, KV head)'s K and V exactly once per launch and keeps all G * T query rows of
// that KV head (GQA, Section 3.2) on the same bytes.
//
// Work decomposition: grid (split, KV head, sequence); 4 waves per workgroup (one per SIMD);
// each wave takes 32-key chunks of the split round-robin.
//   Prologue: the workgroup translates the split's keys into physical cache rows once (block
//     table, and for a draft the selection list) into an LDS table, so no dependent global
//     read sits in front of a K/V load in the main loop. For a draft the selection-list reads
//     do not wait for the sequence's lengths: the prologue costs two round trips (lengths,
//     list and queries together; then the block table).
//   Main loop, register double-buffered: the K and V rows of the wave's next chunk are in
//     flight while the current chunk is computed:
//     S^T (16 keys x 16 rows tiles) = K . Q^T with v_mfma_f32_16x16x32_bf16; K rows come from
//       HBM as the A operand (16 B per lane, one key row per 16 lanes); Q^T stays resident in
//       registers as the B operand;
//     online softmax in the log2 domain (row max across the 4 lane groups with xor shuffles;
//       each lane owns one query row of the C tile);
//     O^T (16 dims x 16 rows) += V^T . P^T with P split into bf16 hi + lo parts so that P
//       carries ~16 mantissa bits: two MFMAs, or, when the tile has room for twice the query
//       rows (R <= 8: a draft, or a one-token decode), one MFMA whose rows R .. 2R - 1 repeat
//       the queries and carry the lo parts; V^T is read transposed from a padded LDS tile that
//       the same wave wrote: V rows arrive with row-contiguous nontemporal loads (each
//       instruction covers whole rows, the pattern that keeps the HBM read rate highest); K
//       rows, used straight from registers as the MFMA operand, keep plain loads (routing K
//       through LDS as well measured slower).
// Waves merge (max, sum, O) through LDS; with one split the workgroup writes the final
// normalised output, otherwise (m, l, o) partials that the merge kernel combines.
// Over the full cache, sequences are taken longest first (see the kernel's prologue).

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kWaves = 4;
constexpr unsigned kInvalidRow = 0xffffffffu;
// Largest batch whose workgroups order themselves longest-first (each ranks every sequence:
// O(B^2 / 64) work per workgroup).
constexpr int kLongestFirstMaxBatch = 256;
// Table entries each thread of a draft workgroup fills per pass (1024 keys per pass: one pass
// covers a draft set of up to 1024 keys per split).
constexpr int kSelUnroll = 4;

template <int D, int NRT>
struct MfmaCfg {
    static constexpr int KS = D / 32;          // k-steps of the QK^T contraction
    static constexpr int DT = D / 16;          // dim tiles of the PV product
    static constexpr int ROWS = 16 * NRT;      // query rows held per wave
    static constexpr int STRIDE = D + 4;       // LDS row stride in bf16 (row = D/2 + 2 dwords)
    static constexpr int VLDS = kWaves * 32 * STRIDE * 2;            // bytes
    static constexpr int TAB = (kMfmaTableEntries + 1) * 4;          // bytes
    static constexpr int MERGE = kWaves * ROWS * (D + 2) * 4;        // bytes
    static constexpr int SMEM = (VLDS + TAB) > MERGE ? (VLDS + TAB) : MERGE;
};

// Entries of the physical-row table one thread fills per pass of the dense prologue; their
// global reads are all issued before any is waited on.
constexpr int kTabUnroll = 4;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
    bf16x8 r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

// Workgroups are dispatched in grid order, so the z-th row of the grid taking the sequence of
// rank z in decreasing length (ties: lower index) starts the longest sequences first and ends a
// ragged batch with short ones instead of a long tail. Every wave computes the same answer
// from one vector load of the lengths per 64 sequences, with no LDS or barrier; a batch of
// equal lengths keeps z (the wave-uniform min == max test) and skips the ranking.
__device__ __forceinline__ int longest_first(const AttnArgs& a, int z, int lane) {
    constexpr int kChunks = kLongestFirstMaxBatch / 64;
    int len[kChunks];
    int lo = 0x7fffffff, hi = -1;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int j = c * 64 + lane;
        len[c] = -1;
        if (c * 64 < a.B && j < a.B) {
            len[c] = max(min(a.kv_lens[j], a.max_kv_len), 0);
            lo = min(lo, len[c]);
            hi = max(hi, len[c]);
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lo = min(lo, __shfl_xor(lo, o));
        hi = max(hi, __shfl_xor(hi, o));
    }
    if (__builtin_amdgcn_readfirstlane(lo) == __builtin_amdgcn_readfirstlane(hi)) return z;
    int found = -1;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c * 64 >= a.B) break;
        const int j = c * 64 + lane;
        int rank = 0;
#pragma unroll
        for (int c2 = 0; c2 < kChunks; ++c2) {
            if (c2 * 64 >= a.B) break;
            const int n = min(64, a.B - c2 * 64);
            for (int t = 0; t < n; ++t) {
                const int Li = __builtin_amdgcn_readlane(len[c2], t);
                rank += (Li > len[c] || (Li == len[c] && c2 * 64 + t < j)) ? 1 : 0;
            }
        }
        if (j < a.B && rank == z) found = j;
    }
    const unsigned long long hit = __ballot(found >= 0);       // exactly one lane
    return hit != 0ull ? __builtin_amdgcn_readlane(found, __ffsll((long long)hit) - 1) : z;
}

// Cross-wave merge of one workgroup's results: every wave left its (max, sum) per row in sml
// ([wave][ROWS][2]) and its O rows in so ([wave][ROWS][D]); with one split the normalised
// output (and LSE) is written, otherwise the (m, l, o) partial of `split`. Each thread merges 4
// consecutive dims of one row per step: the waves' (m, l) of the row as four 8-byte reads,
// their outputs as 16-byte reads, the result as 16-byte (output) or 8-byte (split partial)
// stores.
template <int D, int NRT, bool FOLD>
__device__ __forceinline__ void merge_out(const AttnArgs& a, const float* so, const float* sml,
                                          int nlast, int b, int g, int split, bool poisoned,
                                          int tid) {
    constexpr int ROWS = 16 * NRT;
    const float qnan = __builtin_nanf("");
    constexpr int D4 = D / 4;
    const float2* sml2 = reinterpret_cast<const float2*>(sml);  // (m, l) of [wave][row]
    const bool out16 = (reinterpret_cast<uintptr_t>(a.out) & 15) == 0;
    const bool part8 = (reinterpret_cast<uintptr_t>(a.part) & 7) == 0;
    for (int idx = tid; idx < a.R * D4; idx += kWaves * 64) {
        const int r = idx / D4, d = (idx % D4) * 4;
        float2 ml[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ml[w] = sml2[w * ROWS + r];
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[w].x);
        float lsum = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float e = __builtin_amdgcn_exp2f(ml[w].x - M);
                float4 ow = *reinterpret_cast<const float4*>(so + (w * ROWS + r) * D + d);
                if (FOLD && r >= 16 * (NRT - 1)) {
                    const float4 lo = *reinterpret_cast<const float4*>(so + (w * ROWS + r + nlast) * D + d);
                    ow.x += lo.x; ow.y += lo.y; ow.z += lo.z; ow.w += lo.w;
                }
                lsum += e * ml[w].y;
                o0 += e * ow.x;
                o1 += e * ow.y;
                o2 += e * ow.z;
                o3 += e * ow.w;
            }
        }
        const int h = g * a.G + r / a.T, t = r % a.T;
        const size_t row = ((size_t)b * a.Hq + h) * a.T + t;
        if (a.nsplit == 1) {
            float4 ov = lsum > 0.f ? make_float4(o0 / lsum, o1 / lsum, o2 / lsum, o3 / lsum)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            if (poisoned) ov = make_float4(qnan, qnan, qnan, qnan);
            float* dst = a.out + row * D + d;
            if (out16) {
                *reinterpret_cast<float4*>(dst) = ov;
            } else {
                dst[0] = ov.x; dst[1] = ov.y; dst[2] = ov.z; dst[3] = ov.w;
            }
            if (d == 0 && a.lse != nullptr) {
                float lv = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : kNegInf;
                a.lse[row] = poisoned ? qnan : lv;
            }
        } else {
            // a partial is D + 2 floats: 8-byte aligned when the workspace is
            float* pp = a.part + (row * a.nsplit + split) * (D + 2);
            const float2 p01 = poisoned ? make_float2(qnan, qnan) : make_float2(o0, o1);
            const float2 p23 = poisoned ? make_float2(qnan, qnan) : make_float2(o2, o3);
            if (part8) {
                *reinterpret_cast<float2*>(pp + d) = p01;
                *reinterpret_cast<float2*>(pp + d + 2) = p23;
            } else {
                pp[d] = p01.x; pp[d + 1] = p01.y; pp[d + 2] = p23.x; pp[d + 3] = p23.y;
            }
            if (d == 0) {
                pp[D] = poisoned ? qnan : M;
                pp[D + 1] = poisoned ? qnan : lsum;
            }
        }
    }
}

// With one row tile the kernel fits two workgroups per CU (<= 256 registers per lane), so a
// draft launch of B * Hkv workgroups is resident in a single round. FOLD (the last row tile
// holds n <= 8 of the R query rows) puts the lo parts of that tile's P in its rows n .. 2n - 1
// instead of a second MFMA: a draft's 4 rows, or a verify's rows 16 .. R - 1 for R <= 24.
template <int D, bool GATHER, int NRT, bool FOLD>
__global__ __launch_bounds__(kWaves * 64, NRT == 1 ? 2 : 1) void attn_mfma_kernel(AttnArgs a) {
    using C = MfmaCfg<D, NRT>;
    constexpr int NBUF = 2;            // chunks in flight per wave
    constexpr int KS = C::KS, DT = C::DT, STRIDE = C::STRIDE, ROWS = C::ROWS;
    constexpr int kLPR = D / 8;            // lanes per V row (16 B each)
    constexpr int kRPI = 64 / kLPR;        // V rows per load instruction (KS * kRPI = 16)
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int split = blockIdx.x, g = blockIdx.y;
    if (tid == 0) s_bad = 0;
    // Sequence of this workgroup: over the full cache (work proportional to the length) a
    // ragged batch is taken longest first (see longest_first).
    int b = blockIdx.z;
    if constexpr (!GATHER) {
        if (a.B > 1 && a.B <= kLongestFirstMaxBatch) b = longest_first(a, blockIdx.z, lane);
    }
    const int v_begin = split * a.split_len;
    const int32_t* sel = GATHER ? a.sel_idx + ((size_t)b * a.Hkv + g) * a.k_max : nullptr;
    const int32_t* btab = a.block_table + (size_t)b * a.max_blocks;
    unsigned* rowtab = reinterpret_cast<unsigned*>(smem + C::VLDS);

    // Draft prologue: the first pass of selection entries, the queries and the sequence's
    // lengths are all requested before any of them is waited for, so together they cost one
    // round trip (the block-table reads that depend on them are the second). Entry v < k_max is
    // read whatever the count turns out to be; whether it is listed is decided once the count
    // is known.
    int sv0[GATHER ? kSelUnroll : 1];
    if constexpr (GATHER) {
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
            const int v = v_begin + u * kWaves * 64 + tid;
            sv0[u] = v < a.k_max ? sel[v] : 0;
        }
    }

    // Q^T as the B operand: lane supplies column (row) rt*16 + m16, dims ks*32 + q4*8 .. +7.
    // Folded: in the last tile, with n = R - 16 (NRT - 1) rows, columns n .. 2n - 1 repeat
    // that tile's rows 0 .. n - 1. (Issued with the prologue's other loads: the queries do
    // not depend on the lengths.)
    const int nlast = a.R - 16 * (NRT - 1);     // query rows in the last tile
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    bf16x8 qop[NRT][KS];
    int qrow[NRT];                     // query row of this lane's column, or -1
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        int r = rt * 16 + m16;
        if (FOLD && rt == NRT - 1 && m16 >= nlast && m16 < 2 * nlast) r -= nlast;
        qrow[rt] = r < a.R ? r : -1;
        if (r < a.R) {
            const int h = g * a.G + r / a.T, t = r % a.T;
            const uint16_t* src = qp + (((size_t)b * a.Hq + h) * a.T + t) * D + q4 * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qop[rt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(src + ks * 32));
        } else {
            // zero queries: finite scores, never written out, and no causal bound
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qop[rt][ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }

    // The sequence's lengths. For a draft, lanes 0, 1, 2 fetch them with one vector load issued
    // after the loads above, so one wait covers all of them (plain uniform loads would be scalar
    // loads, which the compiler issues only after waiting for the vector loads: a second round
    // trip).
    int L, n_list = 0, lo = 0;
    if constexpr (GATHER) {
        const int32_t* lp = lane == 0 ? a.kv_lens : (lane == 1 ? a.sel_count : a.tail_lo);
        const int x = lane < 3 ? lp[b] : 0;
        L = __builtin_amdgcn_readlane(x, 0);
        n_list = __builtin_amdgcn_readlane(x, 1);
        lo = __builtin_amdgcn_readlane(x, 2);
        L = max(min(L, a.max_kv_len), 0);
        n_list = min(max(n_list, 0), a.k_max);
        lo = min(max(lo, 0), L);
    } else {
        L = max(min(a.kv_lens[b], a.max_kv_len), 0);
    }
    const int total = n_list + (L - lo);
    const int v_end = (split == a.nsplit - 1) ? total : min(v_begin + a.split_len, total);

    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v);
    const int bs = a.bs, sh = (bs & (bs - 1)) == 0 ? __builtin_ctz(bs) : -1;

    int limit[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
        limit[rt] = (GATHER || qrow[rt] < 0) ? 0x7fffffff : L - a.T + qrow[rt] % a.T;
    // Every key below this position is visible to every query row (the first causal row).
    const int lim_all = GATHER ? 0x7fffffff : L - a.T;
    // Folded: lanes of the last tile's rows n .. 2n - 1 feed the lo parts of P to the PV product.
    const bool lo_lane = FOLD && m16 >= nlast && m16 < 2 * nlast;

    f32x4 o[DT][NRT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow[NRT], lrow[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) { mrow[rt] = kNegInf; lrow[rt] = 0.f; }

    uint16_t* vl = reinterpret_cast<uint16_t*>(smem) + wid * 32 * STRIDE;

    // Draft table fill, one pass: rowtab[i] for i = base + u * 256 + tid (u < kSelUnroll) =
    // physical row of key v = seg + i of [seg, seg_end), from the selection entries sv and the
    // block table. All of a thread's block-table reads are issued before any is used.
    auto fill_gather = [&](int seg, int seg_end, int base, const int (&sv)[kSelUnroll]) {
        const int n = seg_end - seg;
        int pos[kSelUnroll];
        bool ok[kSelUnroll];
        int blk[kSelUnroll];
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
            const int v = seg + base + u * kWaves * 64 + tid;
            const bool listed = v < n_list;
            pos[u] = listed ? sv[u] : lo + (v - n_list);
            ok[u] = v < seg_end && (!listed || (sv[u] >= 0 && sv[u] < lo));
            blk[u] = btab[ok[u] ? div_bs(pos[u], bs, sh) : 0];
        }
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
            const int i = base + u * kWaves * 64 + tid;
            if (i >= n) continue;
            unsigned row = kInvalidRow;
            if (ok[u]) {
                if ((unsigned)blk[u] < (unsigned)a.num_blocks)
                    row = ((unsigned)blk[u] * a.Hkv + g) * bs + (pos[u] - div_bs(pos[u], bs, sh) * bs);
                else
                    s_bad = 1;
            }
            rowtab[i] = row;
        }
    };
    // Later passes of a draft table (sets of more than 1024 keys per split): their selection
    // entries are read in the pass.
    auto fill_rest = [&](int seg, int seg_end, int from) {
        for (int base = from; base < seg_end - seg; base += kSelUnroll * kWaves * 64) {
            int sv[kSelUnroll];
#pragma unroll
            for (int u = 0; u < kSelUnroll; ++u) {
                const int v = seg + base + u * kWaves * 64 + tid;
                sv[u] = v < a.k_max ? sel[v] : 0;
            }
            fill_gather(seg, seg_end, base, sv);
        }
    };
    if constexpr (GATHER) {
        // First segment, first pass: its selection entries are already in registers (they die
        // here, before the main loop).
        __syncthreads();                               // s_bad is initialised
        const int seg_end0 = min(v_begin + kMfmaTableEntries, v_end);
        if (v_begin < v_end) {
            fill_gather(v_begin, seg_end0, 0, sv0);
            fill_rest(v_begin, seg_end0, kSelUnroll * kWaves * 64);
        }
    }

    // Segment = the keys whose rows one LDS table holds (the planner keeps a split to one).
    const int seg_keys = GATHER ? kMfmaTableEntries : kMfmaTableEntries * bs;
    for (int seg = v_begin; seg < v_end; seg += seg_keys) {
        const int seg_end = min(seg + seg_keys, v_end);
        const int blk0 = seg / bs;
        if constexpr (GATHER) {
            if (seg != v_begin) {           // a split longer than one table: refill it
                __syncthreads();            // the previous segment's table is no longer read
                fill_rest(seg, seg_end, 0);
            }
        } else {
            __syncthreads();                // the previous segment's table is no longer read
            const int nblk = (seg_end - 1) / bs - blk0 + 1;
            for (int base = 0; base < nblk; base += kTabUnroll * kWaves * 64) {
                int blk[kTabUnroll];
#pragma unroll
                for (int u = 0; u < kTabUnroll; ++u) {
                    const int i = base + u * kWaves * 64 + tid;
                    blk[u] = i < nblk ? btab[blk0 + i] : 0;
                }
#pragma unroll
                for (int u = 0; u < kTabUnroll; ++u) {
                    const int i = base + u * kWaves * 64 + tid;
                    if (i >= nblk) continue;
                    unsigned row = kInvalidRow;
                    if ((unsigned)blk[u] < (unsigned)a.num_blocks)
                        row = ((unsigned)blk[u] * a.Hkv + g) * bs;
                    else
                        s_bad = 1;
                    rowtab[i] = row;
                }
            }
        }
        __syncthreads();

        // Issue the K/V loads of one 32-key chunk into registers. okm[kt] has bit i set when
        // key c0 + 16 kt + i is a valid cache row. Masked keys load cache row 0 (always a valid
        // address) and are discarded: their scores become -inf and their V rows are zeroed
        // when consumed.
        // K in MFMA operand order: an instruction covers 64 B of each of 16 rows, which plain
        // loads serve best (the caches merge the two halves of a line). V goes through LDS, so
        // it is read row-contiguously: instruction ks covers whole rows kRPI * ks .. + kRPI - 1
        // of the tile with nontemporal loads.
        auto issue = [&](int c0, uint4 (&kr)[2][KS], uint4 (&vr)[2][KS], unsigned (&okm)[2]) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int t0 = c0 + kt * 16;                          // wave-uniform
                if constexpr (GATHER) {
                    const int v = t0 + m16;
                    const unsigned row = v < seg_end ? rowtab[v - seg] : kInvalidRow;
                    const bool ok = row != kInvalidRow;
                    okm[kt] = (unsigned)(__ballot(ok) & 0xffffull);
                    const size_t off = (size_t)(ok ? row : 0u) * D + q4 * 8;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        kr[kt][ks] = *reinterpret_cast<const uint4*>(kp + off + ks * 32);
                        const int j = ks * kRPI + lane / kLPR;
                        const unsigned vrow = (unsigned)__shfl((int)row, j);
                        const bool vok = (okm[kt] >> j) & 1u;
                        vr[kt][ks] = load_stream(vp + (size_t)(vok ? vrow : 0u) * D + (lane % kLPR) * 8);
                    }
                } else {
                    // Chunks start on multiples of 16 and the block size is a multiple of 16,
                    // so the tile's 16 keys are consecutive rows of one block: one uniform
                    // table read gives them all.
                    unsigned r0 = 0;
                    int n_ok = 0;
                    if (t0 < seg_end) {
                        const int blk = div_bs(t0, bs, sh);
                        const unsigned base = __builtin_amdgcn_readfirstlane(rowtab[blk - blk0]);
                        if (base != kInvalidRow) {
                            r0 = base + (unsigned)(t0 - blk * bs);
                            n_ok = min(seg_end - t0, 16);
                        }
                    }
                    okm[kt] = n_ok >= 16 ? 0xffffu : ((1u << n_ok) - 1u);
                    const uint16_t* kq = kp + (size_t)(m16 < n_ok ? r0 + m16 : 0u) * D + q4 * 8;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        kr[kt][ks] = *reinterpret_cast<const uint4*>(kq + ks * 32);
                        const int j = ks * kRPI + lane / kLPR;
                        vr[kt][ks] = load_stream(vp + (size_t)(j < n_ok ? r0 + j : 0u) * D + (lane % kLPR) * 8);
                    }
                }
            }
        };

        // Fold one chunk into the running softmax state.
        auto consume = [&](int c0, uint4 (&kr)[2][KS], uint4 (&vr)[2][KS], unsigned (&okm)[2]) {
            wave_lds_order();
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int j = ks * kRPI + lane / kLPR;           // row of the tile this lane read
                    const bool ok = (okm[kt] >> j) & 1u;
                    *reinterpret_cast<uint4*>(vl + (kt * 16 + j) * STRIDE + (lane % kLPR) * 8) =
                        ok ? vr[kt][ks] : make_uint4(0, 0, 0, 0);
                }
            }

            // S^T = K . Q^T : C tile [key 4*q4+i][row m16].
            f32x4 sacc[2][NRT];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[kt][ks]),
                                                                     qop[rt][ks], acc, 0, 0, 0);
                    sacc[kt][rt] = acc;
                }

            // A full chunk (all 32 keys valid and visible to every row) skips the masks and
            // keeps its reference maximum unless a score exceeds it by more than kLazyMax
            // (log2 units): then p <= 2^kLazyMax, well inside float and the hi + lo split, and
            // O is rescaled only when the maximum has really moved.
            constexpr float kLazyMax = 16.f;
            const bool full = (okm[0] & okm[1]) == 0xffffu && c0 + 31 <= lim_all;
            bf16x8 phi[NRT], plo[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                float sv[8];
                float cmax = kNegInf;
                if (full) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = sacc[kt][rt][i] * a.scale_log2;
                            sv[kt * 4 + i] = x;
                            cmax = fmaxf(cmax, x);
                        }
                } else {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int key = kt * 16 + q4 * 4 + i;
                            bool allowed = (okm[kt] >> (q4 * 4 + i)) & 1u;
                            if constexpr (!GATHER) allowed = allowed && (c0 + key <= limit[rt]);
                            const float x = allowed ? sacc[kt][rt][i] * a.scale_log2 : kNegInf;
                            sv[kt * 4 + i] = x;
                            cmax = fmaxf(cmax, x);
                        }
                }
                cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
                cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
                // the first chunk of a row always moves its maximum (mrow = -inf)
                const bool move = full ? cmax > mrow[rt] + kLazyMax : cmax > mrow[rt];
                if (__ballot(move) != 0ull) {
                    const float mnew = fmaxf(mrow[rt], cmax);
                    const float muse = (mnew == kNegInf) ? 0.f : mnew;
                    const float alpha = __builtin_amdgcn_exp2f(mrow[rt] - muse);
                    mrow[rt] = mnew;
                    lrow[rt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
                }
                const float muse = (mrow[rt] == kNegInf) ? 0.f : mrow[rt];
                float psum = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float p = __builtin_amdgcn_exp2f(sv[j] - muse);
                    const __bf16 hi = (__bf16)p;
                    const __bf16 lo_part = (__bf16)(p - (float)hi);
                    if (FOLD && rt == NRT - 1) {
                        phi[rt][j] = lo_lane ? lo_part : hi;
                    } else {
                        phi[rt][j] = hi;
                        plo[rt][j] = lo_part;
                    }
                    psum += p;
                }
                lrow[rt] += psum;
            }

            // O^T += V^T . P^T. k-slot j of lane group q4 is key 16*(j/4) + 4*q4 + (j%4),
            // matching the C-tile keys this lane holds in sacc[j/4][*][j%4]. The V^T operand
            // comes from the transposing LDS read: in each 16-lane group, lane i receives
            // element i%4 of the 8-byte rows addressed by lanes 4k + i/4 (k = 0..3). Lane s
            // addresses V[key 4*q4 + s/4 (+16)][dt*16 + 4*(s%4)], so lane m receives
            // V[4*q4 + k (+16)][dt*16 + m] for k = 0..3: slots j = 0..3 (and 4..7).
            wave_lds_order();
            const int trow = 4 * q4 + (m16 >> 2), tcol = 4 * (m16 & 3);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vl + trow * STRIDE + dt * 16 + tcol));
                const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vl + (trow + 16) * STRIDE + dt * 16 + tcol));
                uint4 wv;
                __builtin_memcpy(&wv.x, &lo4, 8);
                __builtin_memcpy(&wv.z, &hi4, 8);
                const bf16x8 av = as_bf16x8(wv);
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi[rt], o[dt][rt], 0, 0, 0);
                    if (!FOLD || rt < NRT - 1)
                        o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo[rt], o[dt][rt], 0, 0, 0);
                }
            }
            wave_lds_order();
        };

        // Walk over this wave's chunks with NBUF chunks always in flight: consume buffer i,
        // reissue it NBUF chunks ahead, move to buffer i + 1. Issues are unconditional (a
        // chunk past the end loads a dummy row and is fully masked) and the loop condition is
        // the only exit, so every consume is reached with the same loads outstanding and the
        // compiler's wait covers only the chunk being consumed.
        constexpr int stride = kWaves * 32;
        uint4 kbuf[NBUF][2][KS], vbuf[NBUF][2][KS];
        unsigned okbuf[NBUF][2];
        int c = seg + wid * 32;
#pragma unroll
        for (int i = 0; i < NBUF; ++i) issue(c + i * stride, kbuf[i], vbuf[i], okbuf[i]);
        for (; c < seg_end; c += NBUF * stride) {
#pragma unroll
            for (int i = 0; i < NBUF; ++i) {
                consume(c + i * stride, kbuf[i], vbuf[i], okbuf[i]);
                issue(c + (i + NBUF) * stride, kbuf[i], vbuf[i], okbuf[i]);
            }
        }
    }

    // Row sums were kept per lane group; complete them.
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        lrow[rt] += __shfl_xor(lrow[rt], 16);
        lrow[rt] += __shfl_xor(lrow[rt], 32);
    }

    __syncthreads();                 // every wave is done with its V tile (smem is reused)
    float* so = reinterpret_cast<float*>(smem);               // [wave][ROWS][D]
    float* sml = so + kWaves * ROWS * D;                       // [wave][ROWS][2]
    // Rows that reach the output: R (and, folded, the last tile's lo rows).
    const int live = FOLD ? 16 * (NRT - 1) + 2 * nlast : ROWS;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            if (rt * 16 + m16 < live) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[(wid * ROWS + rt * 16 + m16) * D + dt * 16 + q4 * 4 + i] = o[dt][rt][i];
            }
    if (q4 == 0) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            sml[(wid * ROWS + rt * 16 + m16) * 2 + 0] = mrow[rt];
            sml[(wid * ROWS + rt * 16 + m16) * 2 + 1] = lrow[rt];
        }
    }
    __syncthreads();

    merge_out<D, NRT, FOLD>(a, so, sml, nlast, b, g, split, s_bad != 0, tid);
}

template <int D, int NRT, bool FOLD>
void launch_d(const AttnArgs& a, bool gather, dim3 grid, dim3 block, hipStream_t s) {
    if (gather) attn_mfma_kernel<D, true, NRT, FOLD><<<grid, block, 0, s>>>(a);
    else attn_mfma_kernel<D, false, NRT, FOLD><<<grid, block, 0, s>>>(a);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, bool gather, hipStream_t s) {
    dim3 grid(a.nsplit, a.Hkv, a.B), block(kWaves * 64);
    // one row tile up to 16 rows, else two; the last tile is folded when it holds <= 8 rows
    const bool one = a.R <= 16;
    const bool fold = one ? a.R <= 8 : a.R <= 24;
    if (a.D == 128) {
        if (one) fold ? launch_d<128, 1, true>(a, gather, grid, block, s)
                      : launch_d<128, 1, false>(a, gather, grid, block, s);
        else fold ? launch_d<128, 2, true>(a, gather, grid, block, s)
                  : launch_d<128, 2, false>(a, gather, grid, block, s);
    } else {
        if (one) fold ? launch_d<64, 1, true>(a, gather, grid, block, s)
                      : launch_d<64, 1, false>(a, gather, grid, block, s);
        else fold ? launch_d<64, 2, true>(a, gather, grid, block, s)
                  : launch_d<64, 2, false>(a, gather, grid, block, s);
    }
    return hipGetLastError();
}

}  // namespace kvss
