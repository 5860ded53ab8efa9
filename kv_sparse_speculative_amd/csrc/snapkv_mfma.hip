// bf16 SnapKV score passes on gfx950 matrix cores (MagicDec Section 4.4: static SnapKV
// selection, computed once per prompt at prefill per Appendix A.1 / Fig. 8).
//
// For sequence b, KV head g and the R = G * w observation rows (q-head h of group g, window
// query i at position P - w + i):
//   pass 1 (rowstats): per row the softmax max and sum over its causal range [0, P - w + i];
//   pass 2 (colscore): per candidate key j < P - w, c[j] = sum_rows exp(s_rj - m_r) / l_r.
// Both passes stream K once each from HBM (K rows as 16-byte lane loads, double-buffered in
// registers; physical rows from a per-workgroup LDS table of block bases) and keep the
// observation queries in LDS laid out in MFMA operand order, so every operand read is one
// conflict-free 1 KB ds_read_b128 per wave.
//   pass 1: S^T tile (16 keys x 16 rows) = K . Q^T, K as the A operand. Each lane keeps an
//           online (max, sum) of the scores it holds for its row; the 4 lane groups and the 4
//           waves are merged once at the end.
//   pass 2: S tile (16 rows x 16 keys) = Q . K^T, K as the B operand. Each lane holds 4 rows of
//           one key column, so the column sum is an in-lane sum plus one cross-group reduction.
// Scores use scale * log2(e) in float32 after the bf16 contraction; statistics are kept in the
// log2 domain. Partials are written per split; pass 2 merges them per row in its prologue.

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kW = 4;              // waves per workgroup
constexpr unsigned kBadRow = 0xffffffffu;

__device__ __forceinline__ bf16x8 to_bf16x8(const uint4& u) {
    bf16x8 r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

// Q_obs rows of (b, g) -> LDS in MFMA operand order: entry (tile, ks, lane) holds
// Q[row tile*16 + lane%16][ks*32 + (lane/16)*8 .. +7] (16 B); rows past R are zero.
template <int D>
__device__ void stage_queries(const SnapArgs& a, int b, int g, int NT, uint4* qs) {
    constexpr int KS = D / 32;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_obs);
    for (int e = threadIdx.x; e < NT * KS * 64; e += kW * 64) {
        const int lane = e & 63, ks = (e >> 6) % KS, t = (e >> 6) / KS;
        const int r = t * 16 + (lane & 15);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < a.R) {
            const int h = g * a.G + r / a.w, i = r % a.w;
            v = *reinterpret_cast<const uint4*>(qp + (((size_t)b * a.Hq + h) * a.w + i) * D +
                                                ks * 32 + (lane >> 4) * 8);
        }
        qs[e] = v;
    }
}

// Block bases of the keys [k0, k1) of (b, g) -> LDS; returns false if a block id is invalid.
__device__ bool stage_blocks(const SnapArgs& a, int b, int g, int k0, int k1, unsigned* tab) {
    bool bad = false;
    if (k1 <= k0) return false;
    const int blk0 = k0 / a.bs, nblk = (k1 - 1) / a.bs - blk0 + 1;
    const int32_t* btab = a.block_table + (size_t)b * a.max_blocks;
    for (int i = threadIdx.x; i < nblk; i += kW * 64) {
        const int blk = btab[blk0 + i];
        unsigned row = kBadRow;
        if ((unsigned)blk < (unsigned)a.num_blocks) row = ((unsigned)blk * a.Hkv + g) * a.bs;
        else bad = true;
        tab[i] = row;
    }
    return bad;
}

// Load the K rows of one 32-key chunk (keys c0 .. c0+31, each 16 lanes x 16 B) into registers.
// Keys outside [k0, k1) or with a bad block load row 0 and are reported as masked.
template <int D>
__device__ __forceinline__ void load_k(const uint16_t* kp, const unsigned* tab, int bs, int blk0,
                                       int c0, int k1, int m16, int q4, uint4 (&kr)[2][D / 32],
                                       unsigned (&okm)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const int v = c0 + kt * 16 + m16;
        unsigned row = kBadRow;
        if (v < k1) {
            const unsigned base = tab[v / bs - blk0];
            row = base == kBadRow ? kBadRow : base + (unsigned)(v % bs);
        }
        const bool ok = row != kBadRow;
        okm[kt] = (unsigned)(__ballot(ok) & 0xffffull);
        const size_t off = (size_t)(ok ? row : 0u) * D + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            kr[kt][ks] = *reinterpret_cast<const uint4*>(kp + off + ks * 32);
    }
}

template <int D, int NTMAX>
struct SnapCfg {
    static constexpr int KS = D / 32;
    static constexpr int QS = NTMAX * KS * 64 * 16;               // NTMAX row tiles of queries
    static constexpr int TAB = (kMfmaTableEntries + 1) * 4;
};

// ---------------------------------------------------------------- pass 1: row statistics
template <int D, int NTMAX>
__global__ __launch_bounds__(kW * 64) void snap_rowstats_mfma(SnapArgs a) {
    using C = SnapCfg<D, NTMAX>;
    constexpr int KS = C::KS;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::QS + C::TAB];
    __shared__ float sm[kW][NTMAX * 16], sl[kW][NTMAX * 16];
    __shared__ int s_bad;
    uint4* qs = reinterpret_cast<uint4*>(smem);
    unsigned* tab = reinterpret_cast<unsigned*>(smem + C::QS);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int NT = (a.R + 15) / 16;
    const int k0 = split * a.split_len1;
    const int k1 = (split == a.nsplit1 - 1) ? P : min(k0 + a.split_len1, P);
    if (tid == 0) s_bad = 0;
    stage_queries<D>(a, b, g, NT, qs);
    __syncthreads();
    const int blk0 = k0 / a.bs;
    // The planner keeps a split within one table; a longer one is refused (poisoned, not read).
    const bool fits = (k1 - k0) <= (kMfmaTableEntries - 1) * a.bs;
    if (fits) {
        if (stage_blocks(a, b, g, k0, k1, tab)) s_bad = 1;
    } else if (tid == 0) {
        s_bad = 1;
    }
    const int kend = fits ? k1 : k0;
    __syncthreads();

    // Per lane: online (max, sum) of the scores it holds for row t*16 + m16, tile t < NT.
    float mr[NTMAX], lr[NTMAX];
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) { mr[t] = kNegInf; lr[t] = 0.f; }
    // Causal bound of row r: P - w + (r % w).
    int lim[NTMAX];
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) lim[t] = P - a.w + ((t * 16 + m16) % a.w);

    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const int causal_from = P - a.w;            // keys below it are visible to every row

    auto consume = [&](int c0, uint4 (&kr)[2][KS], unsigned (&okm)[2]) {
        const bool full = (okm[0] & okm[1]) == 0xffffu && c0 + 31 < causal_from;
#pragma unroll
        for (int t = 0; t < NTMAX; ++t) {
            if (t >= NT) break;
            uint4 qb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qb[ks] = qs[(t * KS + ks) * 64 + lane];
            float sv[8];
            float cmax = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(kr[kt][ks]),
                                                                 to_bf16x8(qb[ks]), acc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = acc[i] * a.scale_log2;
                    if (!full) {
                        const int key = kt * 16 + q4 * 4 + i;
                        const bool ok = ((okm[kt] >> (q4 * 4 + i)) & 1u) && (c0 + key <= lim[t]);
                        x = ok ? x : kNegInf;
                    }
                    sv[kt * 4 + i] = x;
                    cmax = fmaxf(cmax, x);
                }
            }
            const float mnew = fmaxf(mr[t], cmax);
            if (mnew != kNegInf) {
                float s = lr[t] * __builtin_amdgcn_exp2f(mr[t] - mnew);
#pragma unroll
                for (int j = 0; j < 8; ++j) s += __builtin_amdgcn_exp2f(sv[j] - mnew);
                lr[t] = s;
                mr[t] = mnew;
            }
        }
    };

    constexpr int stride = kW * 32;
    uint4 kA[2][KS], kB[2][KS];
    unsigned okA[2], okB[2];
    int c = k0 + wid * 32;
    load_k<D>(kp, tab, a.bs, blk0, c, kend, m16, q4, kA, okA);
    for (; c < kend; c += 2 * stride) {
        load_k<D>(kp, tab, a.bs, blk0, c + stride, kend, m16, q4, kB, okB);
        consume(c, kA, okA);
        if (c + stride >= kend) break;
        load_k<D>(kp, tab, a.bs, blk0, c + 2 * stride, kend, m16, q4, kA, okA);
        consume(c + stride, kB, okB);
    }

    // Merge the 4 lane groups (xor 16, 32) and then the waves, per row.
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) {
        if (t >= NT) break;
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            const float m2 = __shfl_xor(mr[t], o), l2 = __shfl_xor(lr[t], o);
            const float M = fmaxf(mr[t], m2);
            if (M != kNegInf) {
                lr[t] = lr[t] * __builtin_amdgcn_exp2f(mr[t] - M) + l2 * __builtin_amdgcn_exp2f(m2 - M);
                mr[t] = M;
            }
        }
        if (q4 == 0) { sm[wid][t * 16 + m16] = mr[t]; sl[wid][t * 16 + m16] = lr[t]; }
    }
    __syncthreads();
    const bool poisoned = s_bad != 0;
    for (int r = tid; r < a.R; r += kW * 64) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kW; ++w) M = fmaxf(M, sm[w][r]);
        float L = 0.f;
        if (M != kNegInf)
#pragma unroll
            for (int w = 0; w < kW; ++w) L += sl[w][r] * __builtin_amdgcn_exp2f(sm[w][r] - M);
        float* pp = a.part1 + ((((size_t)b * a.Hkv + g) * a.R + r) * a.nsplit1 + split) * 2;
        pp[0] = poisoned ? __builtin_nanf("") : M;
        pp[1] = poisoned ? __builtin_nanf("") : L;
    }
}

// ---------------------------------------------------------------- pass 2: column scores
template <int D, int NTMAX>
__global__ __launch_bounds__(kW * 64) void snap_colscore_mfma(SnapArgs a) {
    using C = SnapCfg<D, NTMAX>;
    constexpr int KS = C::KS;
    constexpr int TAB = (kSnapColKeys / 16 + 2) * 4;        // block bases of kSnapColKeys keys
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::QS + TAB];
    __shared__ __attribute__((aligned(16))) float rowc[NTMAX * 16];
    __shared__ int s_bad;
    uint4* qs = reinterpret_cast<uint4*>(smem);
    unsigned* tab = reinterpret_cast<unsigned*>(smem + C::QS);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int n = max(P - a.w, 0);
    const int k0 = tile * kSnapColKeys;
    if (k0 >= n) return;
    const int k1 = min(k0 + kSnapColKeys, n);
    const int NT = (a.R + 15) / 16;
    if (tid == 0) s_bad = 0;
    // A operand of S = Q . K^T: lane supplies row m16 of the tile and dims q4*8.. of k-step ks,
    // which is exactly the operand-order staging used for the B operand of pass 1.
    stage_queries<D>(a, b, g, NT, qs);
    for (int r = tid; r < NTMAX * 16; r += kW * 64) {
        float cr = __builtin_huge_valf();          // rows past R (or with no keys) add nothing
        if (r < a.R) {
            const float* pp = a.part1 + (((size_t)b * a.Hkv + g) * a.R + r) * a.nsplit1 * 2;
            float M = kNegInf;
            bool nan = false;
            for (int s = 0; s < a.nsplit1; ++s) { nan |= pp[2 * s] != pp[2 * s]; M = fmaxf(M, pp[2 * s]); }
            float lam = 0.f;
            if (M != kNegInf)
                for (int s = 0; s < a.nsplit1; ++s)
                    if (pp[2 * s] != kNegInf) lam += __builtin_amdgcn_exp2f(pp[2 * s] - M) * pp[2 * s + 1];
            cr = nan ? __builtin_nanf("") : (lam > 0.f ? M + __log2f(lam) : __builtin_huge_valf());
        }
        rowc[r] = cr;
    }
    if (stage_blocks(a, b, g, k0, k1, tab)) s_bad = 1;
    __syncthreads();

    const int blk0 = k0 / a.bs;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    float* dst = a.scores + ((size_t)b * a.Hkv + g) * a.n_stride;
    const bool poisoned = s_bad != 0;

    auto consume = [&](int c0, uint4 (&kr)[2][KS], unsigned (&okm)[2]) {
        float col[2] = {0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NTMAX; ++t) {
            if (t >= NT) break;
            uint4 qa[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[ks] = qs[(t * KS + ks) * 64 + lane];
            const float4 rc = *reinterpret_cast<const float4*>(&rowc[t * 16 + q4 * 4]);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(qa[ks]),
                                                                 to_bf16x8(kr[kt][ks]), acc, 0, 0, 0);
                col[kt] += __builtin_amdgcn_exp2f(acc[0] * a.scale_log2 - rc.x) +
                           __builtin_amdgcn_exp2f(acc[1] * a.scale_log2 - rc.y) +
                           __builtin_amdgcn_exp2f(acc[2] * a.scale_log2 - rc.z) +
                           __builtin_amdgcn_exp2f(acc[3] * a.scale_log2 - rc.w);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            col[kt] += __shfl_xor(col[kt], 16);
            col[kt] += __shfl_xor(col[kt], 32);
            const int key = c0 + kt * 16 + m16;
            if (q4 == 0 && key < k1) {
                const bool ok = (okm[kt] >> m16) & 1u;
                dst[key] = (poisoned || !ok) ? __builtin_nanf("") : col[kt];
            }
        }
    };

    constexpr int stride = kW * 32;
    uint4 kA[2][KS], kB[2][KS];
    unsigned okA[2], okB[2];
    int c = k0 + wid * 32;
    load_k<D>(kp, tab, a.bs, blk0, c, k1, m16, q4, kA, okA);
    for (; c < k1; c += 2 * stride) {
        load_k<D>(kp, tab, a.bs, blk0, c + stride, k1, m16, q4, kB, okB);
        consume(c, kA, okA);
        if (c + stride >= k1) break;
        load_k<D>(kp, tab, a.bs, blk0, c + 2 * stride, k1, m16, q4, kA, okA);
        consume(c + stride, kB, okB);
    }
}

template <int D, int NTMAX>
hipError_t launch_passes(const SnapArgs& a, hipStream_t s) {
    snap_rowstats_mfma<D, NTMAX><<<dim3(a.nsplit1, a.Hkv, a.B), kW * 64, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_stride == 0) return e;
    const dim3 grid((a.n_stride + kSnapColKeys - 1) / kSnapColKeys, a.Hkv, a.B);
    snap_colscore_mfma<D, NTMAX><<<grid, kW * 64, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_snapkv_mfma_passes(const SnapArgs& a, hipStream_t s) {
    const bool small = a.R <= 128;
    if (a.D == 128) return small ? launch_passes<128, 8>(a, s) : launch_passes<128, 16>(a, s);
    return small ? launch_passes<64, 8>(a, s) : launch_passes<64, 16>(a, s);
}

}  // namespace kvss
