// SnapKV selection of the static draft cache (MagicDec Section 4.4: static KV selection,
// computed once at prefill per Appendix A.1 / Fig. 8; budgets in Section 5.2).
//
// Three kernels:
//   rowstats : per observation row (q-head h of group g, window query i) the softmax max and
//              sum over its causal key range [0, P - w + i], split over key ranges;
//   colscore : per candidate key j < P - w, c[j] = sum over the G * w rows of
//              exp(s_rj - m_r) / l_r, with the row statistics merged from the splits;
//   topk     : centred max-pool of c, then an exact radix select of the k-th largest pooled
//              value on its IEEE bit pattern (scores are >= +0, so the bits order like the
//              values) and an ordered compaction (ties go to the lower position), giving the
//              kept positions in ascending order.
// The score passes run on the vector ALU with the queries staged in LDS; they are
// bit-deterministic (fixed key order per thread, no atomics on floats).

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

template <typename ST>
__device__ __forceinline__ float load_elem(const ST* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

template <typename ST, int D>
__global__ __launch_bounds__(256) void snap_rowstats_kernel(SnapArgs a) {
    __shared__ float kt[32][D + 1];
    __shared__ long long soff[32];
    __shared__ int sok[32];
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int begin = split * a.split_len1;
    const int end = (split == a.nsplit1 - 1) ? P : min(begin + a.split_len1, P);
    const PagedCache cache{a.block_table, a.Hkv, a.bs, a.max_blocks, a.num_blocks, D};
    const ST* kp = static_cast<const ST*>(a.k);
    const ST* qp = static_cast<const ST*>(a.q_obs);

    const bool row_ok = tid < a.R;
    const int h = g * a.G + (row_ok ? tid / a.w : 0), i = row_ok ? tid % a.w : 0;
    const int limit = P - a.w + i;
    float q[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        q[d] = row_ok ? load_elem(qp, (((size_t)b * a.Hq + h) * a.w + i) * D + d) : 0.f;
    float m = kNegInf, l = 0.f;
    bool bad = false;

    for (int c0 = begin; c0 < end; c0 += 32) {
        if (tid < 32) {
            const int pos = c0 + tid;
            bool ok = pos < end;
            size_t off = 0;
            if (ok && !cache.row_offset(b, g, pos, off)) { bad = true; ok = false; }
            sok[tid] = ok;
            soff[tid] = (long long)off;
        }
        __syncthreads();
        for (int idx = tid; idx < 32 * D; idx += 256) {
            const int j = idx / D, d = idx % D;
            kt[j][d] = sok[j] ? load_elem(kp, (size_t)soff[j] + d) : 0.f;
        }
        __syncthreads();
        if (row_ok) {
            for (int j = 0; j < 32; ++j) {
                const int pos = c0 + j;
                if (!sok[j] || pos > limit) continue;
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) s = fmaf(q[d], kt[j][d], s);
                s *= a.scale_log2;
                const float mnew = fmaxf(m, s);
                l = l * __builtin_amdgcn_exp2f(m - mnew) + __builtin_amdgcn_exp2f(s - mnew);
                m = mnew;
            }
        }
        __syncthreads();
    }
    const bool poisoned = __syncthreads_or(bad);
    if (row_ok) {
        float* pp = a.part1 + ((((size_t)b * a.Hkv + g) * a.R + tid) * a.nsplit1 + split) * 2;
        pp[0] = poisoned ? __builtin_nanf("") : m;
        pp[1] = poisoned ? __builtin_nanf("") : l;
    }
}

// Rows of the observation window staged in LDS at a time.
template <typename ST>
struct RowChunk { static constexpr int value = sizeof(ST) == 2 ? 128 : 64; };

template <typename ST, int D>
__global__ __launch_bounds__(256) void snap_colscore_kernel(SnapArgs a) {
    constexpr int RC = RowChunk<ST>::value;
    __shared__ __attribute__((aligned(16))) ST qs[RC * D];
    __shared__ float rowc[256];
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int n = max(P - a.w, 0);
    const int j0 = tile * 256;
    if (j0 >= n) return;
    const ST* qp = static_cast<const ST*>(a.q_obs);

    for (int r = tid; r < a.R; r += 256) {
        const float* pp = a.part1 + (((size_t)b * a.Hkv + g) * a.R + r) * a.nsplit1 * 2;
        float M = kNegInf;
        bool nan = false;
        for (int s = 0; s < a.nsplit1; ++s) { nan |= pp[2 * s] != pp[2 * s]; M = fmaxf(M, pp[2 * s]); }
        float lam = 0.f;
        if (M != kNegInf)
            for (int s = 0; s < a.nsplit1; ++s)
                if (pp[2 * s] != kNegInf) lam += __builtin_amdgcn_exp2f(pp[2 * s] - M) * pp[2 * s + 1];
        // log2 of the row normaliser; rows with no visible key contribute nothing.
        rowc[r] = nan ? __builtin_nanf("") : (lam > 0.f ? M + __log2f(lam) : __builtin_huge_valf());
    }

    const int j = j0 + tid;
    const PagedCache cache{a.block_table, a.Hkv, a.bs, a.max_blocks, a.num_blocks, D};
    size_t off = 0;
    const bool live = j < n;
    const bool ok = live && cache.row_offset(b, g, j, off);
    const ST* kp = static_cast<const ST*>(a.k);
    float kr[D];
#pragma unroll
    for (int d = 0; d < D; ++d) kr[d] = ok ? load_elem(kp, off + d) : 0.f;
    float c = 0.f;
    for (int r0 = 0; r0 < a.R; r0 += RC) {
        const int rn = min(RC, a.R - r0);
        __syncthreads();
        for (int idx = tid; idx < rn * D; idx += 256) {
            const int r = r0 + idx / D, d = idx % D;
            const int h = g * a.G + r / a.w, i = r % a.w;
            qs[idx] = qp[(((size_t)b * a.Hq + h) * a.w + i) * D + d];
        }
        __syncthreads();
        for (int rr = 0; rr < rn; ++rr) {
            const ST* qr = qs + (size_t)rr * D;
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) s = fmaf(load_elem(qr, d), kr[d], s);
            c += __builtin_amdgcn_exp2f(s * a.scale_log2 - rowc[r0 + rr]);
        }
    }
    if (live) a.scores[((size_t)b * a.Hkv + g) * a.n_stride + j] = ok ? c : __builtin_nanf("");
}

// Exclusive prefix sum over the 1024 threads of a workgroup; also returns the total.
__device__ int block_scan_1024(int v, int* sh, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < 16; ++w) { run += sh[w]; sh[w] = run; }
    }
    __syncthreads();
    const int base = wid > 0 ? sh[wid - 1] : 0;
    total = sh[15];
    __syncthreads();
    return base + x - v;
}

// Adds one to bin `bin` of `hist` for every lane with `match`: eight ballots give each lane the
// set of lanes holding the same digit and the lowest of them adds the set's size, one LDS atomic
// per distinct digit of the wave (one head's scores share a few exponents, so plain atomics would
// serialise on one bin). Every lane of the wave must call it.
__device__ __forceinline__ void hist_add_wave(unsigned* hist, unsigned bin, bool match, int lane) {
    unsigned long long peers = __ballot(match);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool set = (bin >> bit) & 1u;
        const unsigned long long m = __ballot(set);
        peers &= set ? m : ~m;
    }
    if (match && __ffsll((long long)peers) - 1 == lane)
        atomicAdd(&hist[bin], (unsigned)__popcll(peers));
}

// Radix select (most significant byte first) by the whole block of the k-th largest of the
// values its threads offer through count(prefix, mask, shift, hist), which histograms the digit
// at `shift` of the offered values whose masked bits equal `prefix`. Returns the k-th largest bit
// pattern; `remaining` becomes how many of the values equal to it belong to the k largest.
template <typename CountFn>
__device__ unsigned radix_select_block(unsigned k, unsigned* hist, int* sh, unsigned* s_digit,
                                       unsigned* s_remaining, unsigned& remaining, CountFn count) {
    const int tid = threadIdx.x;
    unsigned prefix = 0, mask = 0;
    remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        count(prefix, mask, shift, hist);
        __syncthreads();
        // the bin where the count from the top first reaches `remaining`
        const int cnt = tid < 256 ? (int)hist[255 - tid] : 0;
        int tot;
        const int above = block_scan_1024(cnt, sh, tot);
        if (tid < 256 && above < (int)remaining && above + cnt >= (int)remaining) {
            *s_digit = 255 - tid;
            *s_remaining = remaining - above;
        }
        __syncthreads();
        prefix |= *s_digit << shift;
        mask |= 255u << shift;
        remaining = *s_remaining;
        __syncthreads();
    }
    return prefix;
}

// Inclusive prefix sum over the 64 lanes of a wave (GFX9 DPP: row shifts, then row broadcasts).
__device__ __forceinline__ unsigned wave_scan_incl(unsigned x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);    // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);    // row_bcast:31
    return x;
}

// Exclusive prefix sum over the 1024 threads of a workgroup with one barrier: every thread adds
// up the wave totals below it itself. `sh` must not be written again until every thread has
// returned.
__device__ __forceinline__ unsigned block_scan_1024_flat(unsigned v, unsigned* sh, unsigned& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const unsigned x = wave_scan_incl(v);
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    unsigned before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const unsigned s = sh[w];
        tot += s;
        before += w < wid ? s : 0u;
    }
    total = tot;
    return before + x - v;
}

// Adds one to bin `bin` of `hist` for every lane with `match`: a single atomic for the wave
// when all matching lanes share the bin (a head's scores share their high digits), one per
// lane otherwise. Every lane of the wave must call it.
__device__ __forceinline__ void hist_add_lanes(unsigned* hist, unsigned bin, bool match, int lane) {
    const unsigned long long act = __ballot(match);
    if (act == 0ull) return;
    const int first = __builtin_ctzll(act);
    const unsigned b0 = __builtin_amdgcn_readlane(bin, first);
    if (__ballot(match && bin != b0) == 0ull) {
        if (lane == first) atomicAdd(&hist[b0], (unsigned)__popcll(act));
    } else if (match) {
        atomicAdd(&hist[bin], 1u);
    }
}

// Every lane of a wave, after the 256-bin histogram (16-byte aligned) is complete: the bin,
// counting from the top, where the running count first reaches `remaining` (which the total
// reaches), and the count still needed inside that bin. Lane l reads bins 252 - 4l .. 255 - 4l.
__device__ __forceinline__ void pick_digit(const unsigned* hist, unsigned remaining, int lane,
                                           unsigned& digit, unsigned& rem_out) {
    const uint4 hv = reinterpret_cast<const uint4*>(hist)[63 - lane];
    const unsigned s = hv.x + hv.y + hv.z + hv.w;
    const unsigned incl = wave_scan_incl(s);
    unsigned acc = incl - s;
    const int at = __builtin_ctzll(__ballot(acc < remaining && incl >= remaining));
    unsigned bin = 255u - 4u * lane;
    if (acc + hv.w < remaining) {
        acc += hv.w; --bin;
        if (acc + hv.z < remaining) {
            acc += hv.z; --bin;
            if (acc + hv.y < remaining) { acc += hv.y; --bin; }
        }
    }
    digit = __builtin_amdgcn_readlane(bin, at);
    rem_out = remaining - __builtin_amdgcn_readlane(acc, at);
}

// End of one radix pass in the one-barrier scheme (every thread of the workgroup calls it): the
// caller has added this pass's digits to hist[hb]; the next buffer is cleared (three rotate, so
// the one cleared was last read two passes ago), the workgroup waits once, and every wave picks
// the digit from hist[hb] itself.
__device__ __forceinline__ void radix_pass_end(unsigned (*hist)[256], int& hb, unsigned& prefix,
                                               unsigned& mask, unsigned& remaining, int shift) {
    const int tid = threadIdx.x;
    const int next = hb == 2 ? 0 : hb + 1;
    if (tid < 64) reinterpret_cast<uint4*>(hist[next])[tid] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    unsigned d, rr;
    pick_digit(hist[hb], remaining, tid & 63, d, rr);
    prefix |= d << shift;
    mask |= 255u << shift;
    remaining = rr;
    hb = next;
}

// Word 3 of a raw buffer resource on gfx9 (32-bit data format); with stride 0 and num_records
// in bytes, an access at or past num_records is dropped (stores) or reads 0 (loads).
constexpr int kBufferWord3 = 0x00020000;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations (lgkmcnt 0) but
// not for its global loads in flight (which __syncthreads() would drain), then joins the barrier.
// It orders nothing in global memory; the compiler still waits for each load before its use.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0); vmcnt and expcnt left as they are
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Prefilter of the generic top-k: candidates held in LDS (bit pattern and position), and the
// number of position groups whose maxima bound the selection from below.
constexpr int kPreCap = 7680;      // 60 KB: the static LDS stays within the default 64 KB
constexpr int kPreGroups = 8192;

__global__ __launch_bounds__(1024) void snap_topk_kernel(SnapArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned hist[3][256];
    __shared__ int sh[16];
    __shared__ unsigned shu[16];
    __shared__ unsigned s_digit, s_remaining;
    __shared__ __attribute__((aligned(16))) unsigned cand_v[kPreCap];
    __shared__ int cand_j[kPreCap];
    __shared__ int wcnt[16];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int n = max(P - a.w, 0);
    const int k = a.keep;
    if (g == 0 && tid == 0) a.sel_count[b] = min(k, n);
    int32_t* out = a.sel_idx + ((size_t)b * a.Hkv + g) * k;
    if (n <= k) {
        for (int j = tid; j < k; j += 1024) out[j] = j < n ? j : -1;
        return;
    }
    const float* c = a.scores + ((size_t)b * a.Hkv + g) * a.n_stride;
    unsigned* pl = reinterpret_cast<unsigned*>(a.pooled + ((size_t)b * a.Hkv + g) * a.n_stride);
    const int r = a.pool / 2;
    if (tid < 64) reinterpret_cast<uint4*>(hist[0])[tid] = make_uint4(0u, 0u, 0u, 0u);
    // Every loop below issues a batch of independent loads before using any (the pooled array
    // is re-read from L2 on every pass; one load at a time would wait out its latency each).
    constexpr int kBatch = 8;
    static_assert(kBatch * 1024 == kPreGroups, "each thread holds kBatch of the j mod kPreGroups groups");
    unsigned gmax[kBatch];       // maximum pooled bit pattern of this thread's groups
#pragma unroll
    for (int q = 0; q < kBatch; ++q) gmax[q] = 0u;
    // Pooling. A neighbour out of [0, n) is -inf; the centre is the score itself.
    constexpr int kTile = 4096, kTileLoads = (kTile + 8 + 1023) / 1024;
    static_assert(kTileLoads * 1024 <= kPreCap, "every staged word lies in the candidate area");
    if (r <= 3) {
        // Tiles of 4096 positions staged through LDS (the candidate area, not yet in use): word
        // i holds position j0 - 4 + i. Thread t pools positions j0 + 4t .. j0 + 4t + 3 from the
        // 12 words 4t .. 4t + 11 (three 16-byte reads) with three-input maxima.
        // Every load of the loop is unconditional, so the compiler counts them and waits for
        // each tile's loads only where they are used. A whole tile's pooled values go out as
        // one 16-byte store per lane (when the row is 16-byte aligned); the tile holding
        // position n - 1 uses buffer stores that the hardware drops past n. The loads of the
        // next kAhead tiles are in flight while one is pooled; the last round may pool up to
        // three tiles past the end, whose stores are all dropped.
        constexpr int kAhead = 4;
        float* tile = reinterpret_cast<float*>(cand_v);
        const int ntiles = (n + kTile - 1) / kTile;
        const __amdgpu_buffer_rsrc_t plr =
            __builtin_amdgcn_make_buffer_rsrc(pl, (short)0, n * 4, kBufferWord3);
        const bool pl16 = (reinterpret_cast<uintptr_t>(pl) & 15) == 0;
        // scores through a buffer resource: positions outside [0, n) read as 0 without an access
        // (a negative position wraps to a huge offset) and are set to -inf in LDS
        const __amdgpu_buffer_rsrc_t cr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(c), (short)0, n * 4, kBufferWord3);
        float v[kAhead][kTileLoads];
        auto load_tile = [&](int t, float (&dst)[kTileLoads]) {
            const int j0 = t * kTile;
#pragma unroll
            for (int q = 0; q < kTileLoads; ++q)
                dst[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       cr, (j0 - 4 + tid + 1024 * q) * 4, 0, 0));
        };
        // group slot of position j0 + 4t + e: 4 (t mod 2) + e, i.e. group j mod kPreGroups
        auto pool_tile = [&](int t, float (&buf)[kTileLoads], auto half) {
            constexpr int H = decltype(half)::value;
            const int j0 = t * kTile;
            lds_barrier();                            // the previous tile's reads are done
#pragma unroll
            for (int q = 0; q < kTileLoads; ++q) tile[tid + 1024 * q] = buf[q];
            if (j0 < 4 || j0 + kTile + 4 > n) {      // the tile reaches past either end
#pragma unroll
                for (int q = 0; q < kTileLoads; ++q) {
                    const int p = j0 - 4 + tid + 1024 * q;
                    if (p < 0 || p >= n) tile[tid + 1024 * q] = kNegInf;
                }
            }
            lds_barrier();
            load_tile(t + kAhead, buf);
            const float4 w0 = reinterpret_cast<const float4*>(tile)[tid];
            const float4 w1 = reinterpret_cast<const float4*>(tile)[tid + 1];
            const float4 w2 = reinterpret_cast<const float4*>(tile)[tid + 2];
            const float w[12] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w2.x, w2.y, w2.z, w2.w};
            // position j0 + 4t + e is w[4 + e]; its window is w[4 + e - r .. 4 + e + r]
            float pm[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float m = w[4 + e];
                if (r >= 1) m = fmaxf(m, fmaxf(w[3 + e], w[5 + e]));
                if (r >= 2) m = fmaxf(m, fmaxf(w[2 + e], w[6 + e]));
                if (r >= 3) m = fmaxf(m, fmaxf(w[1 + e], w[7 + e]));
                pm[e] = m;
            }
            if (j0 + kTile <= n && pl16) {           // a whole tile: one 16-byte store per lane
                *reinterpret_cast<uint4*>(pl + j0 + 4 * tid) =
                    make_uint4(__float_as_uint(pm[0]), __float_as_uint(pm[1]),
                               __float_as_uint(pm[2]), __float_as_uint(pm[3]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pm[e]), plr,
                                                          (j0 + 4 * tid + e) * 4, 0, 0);
            }
            if (j0 + kTile <= n) {
#pragma unroll
                for (int e = 0; e < 4; ++e) gmax[4 * H + e] = max(gmax[4 * H + e], __float_as_uint(pm[e]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gmax[4 * H + e] = max(gmax[4 * H + e], j0 + 4 * tid + e < n ? __float_as_uint(pm[e]) : 0u);
            }
        };
        static_assert(kAhead == 4, "tile t uses buffer t mod 4 and slot half t mod 2");
#pragma unroll
        for (int t = 0; t < kAhead; ++t) load_tile(t, v[t]);
        for (int t = 0; t < ntiles; t += kAhead) {
            pool_tile(t, v[0], std::integral_constant<int, 0>{});
            pool_tile(t + 1, v[1], std::integral_constant<int, 1>{});
            pool_tile(t + 2, v[2], std::integral_constant<int, 0>{});
            pool_tile(t + 3, v[3], std::integral_constant<int, 1>{});
        }
    } else {
        for (int j0 = tid; j0 < n; j0 += kBatch * 1024) {
            float m[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int j = j0 + q * 1024;
                m[q] = j < n ? c[j] : 0.f;
            }
            for (int d = 1; d <= r; ++d) {
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int j = j0 + q * 1024;
                    const float lft = (j < n && j - d >= 0) ? c[j - d] : kNegInf;
                    const float rgt = (j + d < n) ? c[j + d] : kNegInf;
                    m[q] = fmaxf(m[q], fmaxf(lft, rgt));
                }
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int j = j0 + q * 1024;
                if (j < n) {
                    pl[j] = __float_as_uint(m[q]);
                    gmax[q] = max(gmax[q], __float_as_uint(m[q]));
                }
            }
        }
    }
    __syncthreads();

    // Prefilter. The positions fall into kPreGroups groups (j mod kPreGroups); the top 16 bits
    // of the k-th largest group maximum form a bound t0 that at least k pooled values reach, so
    // every value kept is >= t0. When the values >= t0 fit in LDS they are compacted there in
    // position order and the selection runs over them alone; otherwise it runs over the whole
    // pooled array below. Radix passes take one barrier each (radix_pass_end).
    if (k <= kPreGroups / 2) {
        int hb = 0;
        unsigned prefix = 0, mask = 0, remaining = (unsigned)k;
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = 24 - 8 * pass;
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                hist_add_lanes(hist[hb], (gmax[q] >> shift) & 255u, (gmax[q] & mask) == prefix, lane);
            radix_pass_end(hist, hb, prefix, mask, remaining, shift);
        }
        const unsigned t0 = prefix;
        // each wave takes one contiguous span of positions (a multiple of 64): count, then place
        // (16 loads in flight per lane: the pooled array comes back from L2 or the last-level cache)
        constexpr int kScan = 16;
        const int span = (n + 16 * 64 - 1) / (16 * 64) * 64;
        const int w_lo = min(n, wid * span), w_hi = min(n, w_lo + span);
        int cnt = 0;
        for (int j0 = w_lo; j0 < w_hi; j0 += kScan * 64) {
            unsigned uu[kScan];
#pragma unroll
            for (int q = 0; q < kScan; ++q) {
                const int j = j0 + q * 64 + lane;
                const unsigned x = pl[min(j, w_hi - 1)];          // unconditional: no branch
                uu[q] = j < w_hi ? x : 0u;
            }
#pragma unroll
            for (int q = 0; q < kScan; ++q)
                cnt += __popcll(__ballot(j0 + q * 64 + lane < w_hi && uu[q] >= t0));
        }
        if (lane == 0) wcnt[wid] = cnt;
        __syncthreads();
        int off = 0, total = 0;
        for (int w2 = 0; w2 < 16; ++w2) {
            off += w2 < wid ? wcnt[w2] : 0;
            total += wcnt[w2];
        }
        if (total <= kPreCap) {
            for (int j0 = w_lo; j0 < w_hi; j0 += kScan * 64) {
                unsigned uu[kScan];
#pragma unroll
                for (int q = 0; q < kScan; ++q) {
                    const int j = j0 + q * 64 + lane;
                    const unsigned x = pl[min(j, w_hi - 1)];          // unconditional: no branch
                    uu[q] = j < w_hi ? x : 0u;
                }
#pragma unroll
                for (int q = 0; q < kScan; ++q) {
                    const int j = j0 + q * 64 + lane;
                    const bool f = j < w_hi && uu[q] >= t0;
                    const unsigned long long bal = __ballot(f);
                    if (f) {
                        const int o = off + __popcll(bal & ((1ull << lane) - 1ull));
                        cand_v[o] = uu[q];
                        cand_j[o] = j;
                    }
                    off += __popcll(bal);
                }
            }
            __syncthreads();
            prefix = 0;
            mask = 0;
            remaining = (unsigned)k;
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                for (int i0 = 0; i0 < total; i0 += 1024) {       // uniform trip count
                    const int i = i0 + tid;
                    const unsigned u = i < total ? cand_v[i] : 0u;
                    hist_add_lanes(hist[hb], (u >> shift) & 255u, i < total && (u & mask) == prefix,
                                   lane);
                }
                radix_pass_end(hist, hb, prefix, mask, remaining, shift);
            }
            const unsigned thr = prefix;
            // ordered output: thread t takes a contiguous run of the position-ordered
            // candidates; one scan counts, below each thread, the values above thr (low half)
            // and equal to it (high half; total < 2^16)
            const int chunk = (total + 1023) / 1024;
            const int lo = min(total, tid * chunk), hi = min(total, lo + chunk);
            unsigned gt = 0, eq = 0;
            for (int i = lo; i < hi; ++i) { gt += cand_v[i] > thr; eq += cand_v[i] == thr; }
            unsigned tot;
            const unsigned below = block_scan_1024_flat(gt | (eq << 16), shu, tot);
            // values equal to thr taken below this thread (the lowest positions go first)
            const unsigned eq_taken = min(below >> 16, remaining);
            unsigned take = min(remaining - eq_taken, eq);
            unsigned pos = (below & 0xffffu) + eq_taken;
            for (int i = lo; i < hi && pos < (unsigned)k; ++i) {
                const unsigned u = cand_v[i];
                if (u > thr) out[pos++] = cand_j[i];
                else if (u == thr && take > 0) { out[pos++] = cand_j[i]; --take; }
            }
            return;
        }
    }

    // Radix select of the k-th largest bit pattern over the whole pooled array (read from L2 on
    // every pass), when the prefilter does not apply.
    unsigned remaining;
    const int n_pad = (n + 1023) / 1024 * 1024;
    const unsigned thr = radix_select_block(
        (unsigned)k, hist[0], sh, &s_digit, &s_remaining, remaining,
        [&](unsigned prefix, unsigned mask, int shift, unsigned* h) {
            for (int j0 = tid; j0 < n_pad; j0 += kBatch * 1024) {
                unsigned uu[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int j = j0 + q * 1024;
                    uu[q] = j < n ? pl[j] : 0u;
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int j = j0 + q * 1024;
                    if (j0 - tid + q * 1024 >= n_pad) break;      // uniform: whole 1024-blocks
                    hist_add_wave(h, (uu[q] >> shift) & 255u, j < n && (uu[q] & mask) == prefix,
                                  lane);
                }
            }
        });

    const int chunk = (n + 1023) / 1024;
    const int lo = min(n, tid * chunk), hi = min(n, lo + chunk);
    int gt = 0, eq = 0;
    for (int j = lo; j < hi; j += kBatch) {
        unsigned uu[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) uu[q] = j + q < hi ? pl[j + q] : 0u;
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (j + q < hi) { gt += uu[q] > thr; eq += uu[q] == thr; }
    }
    int tot;
    const int eq_before = block_scan_1024(eq, sh, tot);
    int take = min(max((int)remaining - eq_before, 0), eq);
    int pos = block_scan_1024(gt + take, sh, tot);
    for (int j = lo; j < hi && pos < k; j += kBatch) {
        unsigned uu[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) uu[q] = j + q < hi ? pl[j + q] : 0u;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (j + q >= hi || pos >= k) break;
            if (uu[q] > thr) out[pos++] = j + q;
            else if (uu[q] == thr && take > 0) { out[pos++] = j + q; --take; }
        }
    }
}

// Register-resident pool + top-k for up to 1024 * MAXC candidates (MAXC 8, 16 or 32), same
// selection rule as snap_topk_kernel (centred max-pool, k largest by IEEE bits, ties to the
// lower position, ascending output). The kernel is bound by vector instructions per position
// (16 waves share a CU's 4 SIMDs), so every step is kept branch-free and short:
//   1. the scores of one (sequence, KV head) are read once, coalesced, into LDS: position p at
//      word 4 + p + p / MAXC (a pad word after every MAXC, so a thread's run starts at an odd
//      multiple and reading runs is conflict-free; 4 words in front for the first halo);
//   2. thread t owns positions [t*MAXC, t*MAXC + MAXC); it reads them and a halo of kPoolHalo
//      on each side at static offsets from one address (NaN reads as -inf; only the first wave
//      and the waves reaching the end of the range mask by position) and pools them with
//      three-input maxima: every triple, then one more maximum per position;
//   3. prefilter: the positions fall into groups (each thread's run split by position mod 2,
//      else mod 4 or mod 8, the coarsest of these splits that gives at least k non-empty groups).
//      The top 16 bits of the k-th largest group maximum form a bound t0 that at least k pooled
//      values reach, so every kept value is >= t0. The values >= t0 are compacted into LDS in
//      position order and four radix passes over them alone find the k-th largest. A pass is
//      one barrier: the shared 256-bin histogram is filled (one LDS atomic per wave when all
//      its matching lanes share a digit), then every wave picks the digit itself with a DPP
//      scan; histograms rotate over three buffers, so clearing the next one needs no barrier;
//   4. an ordered compaction of the candidates writes the kept positions.
//   Where no split gives k groups, or the values >= t0 do not fit in LDS, steps 3 and 4 run
//   over all pooled values in registers instead (per-wave histograms fed by runs of equal
//   digits, the digit picked with a block scan).
constexpr int kPoolHalo = 3;   // register path: pool kernels up to 2 * kPoolHalo + 1
constexpr int kTopkWaves = 16;
constexpr size_t kTopkMaxLds = 150 * 1024;  // dynamic LDS of the register path (of 160 KB)

// Words of dynamic LDS of the register path: the padded scores of 1024 runs plus the halos.
__host__ __device__ constexpr size_t topk_reg_words(int maxc) { return 1024 * (size_t)(maxc + 1) + 8; }

// Runs of 8 or 16 leave room for two workgroups per CU (37 or 70 KB of LDS) when a wave holds at
// most 64 registers, i.e. eight waves per SIMD.
template <int MAXC>
__global__ __launch_bounds__(1024, MAXC <= 16 ? 8 : 4) void snap_topk_reg_kernel(SnapArgs a) {
    static_assert(MAXC == 8 || MAXC == 16 || MAXC == 32, "run length");
    constexpr int LOG2C = MAXC == 8 ? 3 : MAXC == 16 ? 4 : 5;
    extern __shared__ float lds_scores[];            // padded scores, then candidates or histograms
    __shared__ __attribute__((aligned(16))) unsigned hist[3][256];
    __shared__ unsigned shu[16];
    __shared__ int sh[16];
    __shared__ unsigned s_digit, s_remaining;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int n = max(P - a.w, 0);
    const int k = a.keep;
    if (g == 0 && tid == 0) a.sel_count[b] = min(k, n);
    int32_t* out = a.sel_idx + ((size_t)b * a.Hkv + g) * k;
    if (n <= k) {
        for (int j = tid; j < k; j += 1024) out[j] = j < n ? j : -1;
        return;
    }
    const float* c = a.scores + ((size_t)b * a.Hkv + g) * a.n_stride;
    if (tid < 64) reinterpret_cast<uint4*>(hist[0])[tid] = make_uint4(0u, 0u, 0u, 0u);
    {
        // all of a thread's loads are issued before any is waited on; indices past n re-read
        // the last score (stored beyond the range, never used unmasked)
        float tmp[MAXC];
#pragma clang loop unroll(full)
        for (int q = 0; q < MAXC; ++q) tmp[q] = c[min(tid + q * 1024, n - 1)];
        float* dst = lds_scores + 4 + tid + (tid >> LOG2C);
#pragma clang loop unroll(full)
        for (int q = 0; q < MAXC; ++q) dst[q * (1024 + (1024 >> LOG2C))] = tmp[q];
    }
    __syncthreads();

    const int base = tid * MAXC;
    const int lc = min(max(n - base, 0), MAXC);      // live positions of this thread
    const int r = a.pool / 2;
    // win[q] holds position base - kPoolHalo + q; the pooled value of base + e goes to win[e]
    float win[MAXC + 2 * kPoolHalo];
    {
        const float* src = lds_scores + tid * (MAXC + 1);      // position base - 4 + i at src[i]
        auto word = [](int q) { return q < kPoolHalo ? q : q < MAXC + kPoolHalo ? q + 1 : q + 2; };
        // interior waves: every position of the runs and halos lies in [0, n)
        const bool inner = wid > 0 && (64 * wid + 64) * MAXC + kPoolHalo <= n;
        if (inner) {
#pragma clang loop unroll(full)
            for (int q = 0; q < MAXC + 2 * kPoolHalo; ++q) win[q] = fmaxf(src[word(q)], kNegInf);
        } else {
#pragma clang loop unroll(full)
            for (int q = 0; q < MAXC + 2 * kPoolHalo; ++q) {
                const int p = base - kPoolHalo + q;
                win[q] = (p >= 0 && p < n) ? fmaxf(src[word(q)], kNegInf) : kNegInf;
            }
        }
    }
    {
        float r1[MAXC + 2 * kPoolHalo - 2];           // r1[i]: maximum of win[i .. i + 2]
#pragma clang loop unroll(full)
        for (int i = 0; i < MAXC + 2 * kPoolHalo - 2; ++i)
            r1[i] = fmaxf(fmaxf(win[i], win[i + 1]), win[i + 2]);
        if (r == 0) {
#pragma clang loop unroll(full)
            for (int e = 0; e < MAXC; ++e) win[e] = win[e + 3];
        } else if (r == 1) {
#pragma clang loop unroll(full)
            for (int e = 0; e < MAXC; ++e) win[e] = r1[e + 2];
        } else if (r == 2) {
#pragma clang loop unroll(full)
            for (int e = 0; e < MAXC; ++e) win[e] = fmaxf(r1[e + 1], r1[e + 3]);
        } else {
#pragma clang loop unroll(full)
            for (int e = 0; e < MAXC; ++e) win[e] = fmaxf(fmaxf(r1[e], r1[e + 2]), r1[e + 4]);
        }
    }
    auto live = [&](int e) { return e < lc; };

    // Group maxima by position mod 8 within the run; coarser groups merge them.
    unsigned gm[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma clang loop unroll(full)
    for (int e = 0; e < MAXC; ++e)
        gm[e & 7] = max(gm[e & 7], live(e) ? __float_as_uint(win[e]) : 0u);
    const int tfull = n >> LOG2C, rem = n - (tfull << LOG2C);   // full runs, then the rest
    auto ngroups = [&](int S) { return tfull * S + min(S, rem); };
    // Finer groups give a tighter bound (a pooled maximum repeats over the pool window, so the
    // groups mod 2 already split most repeats) at more values to rank; mod 2 measured best.
    const int S = ngroups(2) >= k ? 2 : ngroups(4) >= k ? 4 : ngroups(8) >= k ? 8 : 0;
    if (S > 0) {
        // group s < S: the positions e of the run with e mod S == s
        unsigned g4[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) g4[s] = max(gm[s], gm[s + 4]);
        const unsigned g2[2] = {max(g4[0], g4[2]), max(g4[1], g4[3])};
        unsigned gs[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) gs[s] = S == 8 ? gm[s] : S == 4 ? g4[s & 3] : g2[s & 1];
        int hb = 0;                                   // histogram buffer of the current pass
        // t0: the top 16 bits of the k-th largest maximum over the non-empty groups
        unsigned prefix = 0, mask = 0, remaining = (unsigned)k;
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = 24 - 8 * pass;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (s < S)
                    hist_add_lanes(hist[hb], (gs[s] >> shift) & 255u,
                                   s < lc && (gs[s] & mask) == prefix, lane);
            radix_pass_end(hist, hb, prefix, mask, remaining, shift);
        }
        const unsigned t0 = prefix;
        unsigned cm = 0;                              // this thread's candidates, bit e
#pragma clang loop unroll(full)
        for (int e = 0; e < MAXC; ++e)
            cm |= (live(e) && __float_as_uint(win[e]) >= t0 ? 1u : 0u) << e;
        unsigned nc;
        unsigned off = block_scan_1024_flat(__popc(cm), shu, nc);
        if (nc <= topk_reg_words(MAXC) / 2) {
            // Every wave is past its pooling reads (the barriers above), so the staged scores
            // can be overwritten: (bit pattern, position) pairs in position order.
            uint2* cand = reinterpret_cast<uint2*>(lds_scores);
#pragma clang loop unroll(full)
            for (int e = 0; e < MAXC; ++e)
                if ((cm >> e) & 1u) cand[off++] = make_uint2(__float_as_uint(win[e]), (unsigned)(base + e));
            __syncthreads();
            prefix = 0;
            mask = 0;
            remaining = (unsigned)k;
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                for (unsigned i0 = 0; i0 < nc; i0 += 1024) {   // uniform trip count
                    const unsigned i = i0 + tid;
                    const unsigned u = i < nc ? cand[i].x : 0u;
                    hist_add_lanes(hist[hb], (u >> shift) & 255u, i < nc && (u & mask) == prefix,
                                   lane);
                }
                radix_pass_end(hist, hb, prefix, mask, remaining, shift);
            }
            const unsigned thr = prefix;
            // ordered output: thread t takes a contiguous run of the candidates; one scan
            // counts, below each thread, the values above thr (low half) and equal to it (high)
            const unsigned chunk = (nc + 1023) / 1024;
            const unsigned lo = min(nc, tid * chunk), hi = min(nc, lo + chunk);
            unsigned gt = 0, eq = 0;
            for (unsigned i = lo; i < hi; ++i) {
                const unsigned u = cand[i].x;
                gt += u > thr;
                eq += u == thr;
            }
            unsigned tot;
            const unsigned below = block_scan_1024_flat(gt | (eq << 16), shu, tot);  // nc < 2^16
            // values equal to thr taken below this thread (the lowest positions go first)
            const unsigned eq_taken = min(below >> 16, remaining);
            unsigned take = min(remaining - eq_taken, eq);
            unsigned pos = (below & 0xffffu) + eq_taken;
            for (unsigned i = lo; i < hi && pos < (unsigned)k; ++i) {
                const uint2 cv = cand[i];
                if (cv.x > thr) out[pos++] = (int)cv.y;
                else if (cv.x == thr && take > 0) { out[pos++] = (int)cv.y; --take; }
            }
            return;
        }
    }

    __syncthreads();                                  // the score staging area is reused below
    unsigned* whist = reinterpret_cast<unsigned*>(lds_scores);      // [kTopkWaves][256]

    unsigned prefix = 0, mask = 0, remaining = (unsigned)k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int t = tid; t < kTopkWaves * 256; t += 1024) whist[t] = 0;
        __syncthreads();
        // A thread's positions are consecutive, and pooled scores of neighbouring positions
        // mostly share their high digits: count runs of one digit in registers and add each
        // run once, so the waves' atomics rarely collide on one histogram word.
        unsigned cur = 0u, run = 0u;
#pragma clang loop unroll(full)
        for (int e = 0; e < MAXC; ++e) {
            const unsigned u = __float_as_uint(win[e]);
            const unsigned bin = (u >> shift) & 255u;
            if (live(e) && (u & mask) == prefix) {
                if (bin != cur && run != 0u) {
                    atomicAdd(&whist[wid * 256 + cur], run);
                    run = 0u;
                }
                cur = bin;
                ++run;
            }
        }
        if (run != 0u) atomicAdd(&whist[wid * 256 + cur], run);
        __syncthreads();
        int cnt = 0;
        if (tid < 256) {
            for (int w = 0; w < kTopkWaves; ++w) cnt += whist[w * 256 + (255 - tid)];
        }
        int tot;
        const int above = block_scan_1024(cnt, sh, tot);
        if (tid < 256 && above < (int)remaining && above + cnt >= (int)remaining) {
            s_digit = 255 - tid;
            s_remaining = remaining - above;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= 255u << shift;
        remaining = s_remaining;
        __syncthreads();
    }
    const unsigned thr = prefix;
    int gt = 0, eq = 0;
#pragma clang loop unroll(full)
    for (int e = 0; e < MAXC; ++e) {
        const unsigned u = __float_as_uint(win[e]);
        gt += live(e) && u > thr;
        eq += live(e) && u == thr;
    }
    int tot;
    const int eq_before = block_scan_1024(eq, sh, tot);
    int take = min(max((int)remaining - eq_before, 0), eq);
    int pos = block_scan_1024(gt + take, sh, tot);
#pragma clang loop unroll(full)
    for (int e = 0; e < MAXC; ++e) {
        const unsigned u = __float_as_uint(win[e]);
        if (!live(e) || pos >= k) continue;
        if (u > thr) out[pos++] = base + e;
        else if (u == thr && take > 0) { out[pos++] = base + e; --take; }
    }
}

template <int MAXC>
hipError_t launch_topk_reg(const SnapArgs& a, dim3 grid, hipStream_t s) {
    const size_t smem = topk_reg_words(MAXC) * 4;
    static_assert(topk_reg_words(32) * 4 <= kTopkMaxLds, "LDS");
    // dynamic LDS beyond the default 64 KB must be allowed per kernel
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&snap_topk_reg_kernel<MAXC>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    snap_topk_reg_kernel<MAXC><<<grid, 1024, smem, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_topk(const SnapArgs& a, hipStream_t s) {
    const dim3 grid(a.Hkv, a.B);
    const int C = (a.n_stride + 1023) / 1024;
    if (a.pool / 2 <= kPoolHalo) {
        if (C <= 8) return launch_topk_reg<8>(a, grid, s);
        if (C <= 16) return launch_topk_reg<16>(a, grid, s);
        if (C <= 32) return launch_topk_reg<32>(a, grid, s);
    }
    snap_topk_kernel<<<grid, 1024, 0, s>>>(a);
    return hipGetLastError();
}

template <typename ST, int D>
hipError_t launch_typed(const SnapArgs& a, hipStream_t s) {
    snap_rowstats_kernel<ST, D><<<dim3(a.nsplit1, a.Hkv, a.B), 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.n_stride > 0) {
        snap_colscore_kernel<ST, D><<<dim3((a.n_stride + 255) / 256, a.Hkv, a.B), 256, 0, s>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_topk(a, s);
}

}  // namespace

hipError_t launch_snapkv(const SnapArgs& a, hipStream_t s) {
    if (a.dtype == 1) {
        // bf16: matrix-core score passes, then pool + top-k.
        hipError_t e = launch_snapkv_mfma_passes(a, s);
        if (e != hipSuccess) return e;
        return launch_topk(a, s);
    }
    return a.D == 128 ? launch_typed<float, 128>(a, s) : launch_typed<float, 64>(a, s);
}

}  // namespace kvss
