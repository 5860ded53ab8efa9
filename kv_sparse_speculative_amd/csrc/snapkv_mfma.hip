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
// conflict-free 1 KB ds_read_b128 per wave. The one-row-tile pass 1 that also stores its scores
// (for a pass 2 that reads them instead of K) loads whole K rows and reorders them in LDS.
//   pass 1: S^T tile (16 keys x 16 rows) = K . Q^T, K as the A operand. Each lane keeps an
//           online (max, sum) of the scores it holds for its row; the 4 lane groups and the 4
//           waves are merged once at the end.
//   pass 2: S tile (16 rows x 16 keys) = Q . K^T, K as the B operand. Each lane holds 4 rows of
//           one key column, so the column sum is an in-lane sum plus one cross-group reduction.
// Scores use scale * log2(e) in float32 after the bf16 contraction; statistics are kept in the
// log2 domain. Partials are written per split; a small kernel between the passes merges them
// into one constant per row, which every pass-2 workgroup of that (sequence, head) reads.
// Each workgroup's prologue issues all of its small loads (block bases, queries, row constants)
// before it waits for any, so it costs one memory round trip before the K stream starts.
// A negative scale is folded into the staged queries (a bf16 sign flip is exact), so the
// kernels only ever multiply by |scale| and the row maximum can be taken before scaling.
// The hot loops are branch-free per lane: every 16-key tile lies in one cache block (splits and
// tiles start on multiples of 16 and the block size is a multiple of 16), so its block lookup
// is wave-uniform.

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kW = 4;              // waves per workgroup
constexpr unsigned kBadRow = 0xffffffffu;
// Word 3 of a raw buffer resource on gfx9 (32-bit data format); with stride 0 and num_records
// in bytes, an access at or past num_records reads 0.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ bf16x8 to_bf16x8(const uint4& u) {
    bf16x8 r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

// Prologue staging, in one memory round trip: the block bases of keys [k0, k1) of (b, g) (TAB
// entries at most), the observation queries of (b, g) in MFMA operand order and, when `rowc` is
// given, the NT * 16 row constants of pass 2. All loads are issued before the first LDS write.
// Query entry (tile, ks, lane) holds Q[row tile*16 + lane%16][ks*32 + (lane/16)*8 .. +7] (16 B);
// rows past R are zero. Returns true if a block id of the range is invalid. The caller follows
// with a barrier.
template <int D, int NT, int TAB>
__device__ bool stage_prologue(const SnapArgs& a, int b, int g, int k0, int k1, unsigned* tab,
                               uint4* qs, const float* rowc, float* rowc_lds) {
    constexpr int KS = D / 32;
    constexpr int NQ = NT * KS * 64;                     // query entries
    constexpr int QPT = (NQ + kW * 64 - 1) / (kW * 64);
    constexpr int TPT = (TAB + kW * 64 - 1) / (kW * 64);
    constexpr int RPT = (NT * 16 + kW * 64 - 1) / (kW * 64);
    const int tid = threadIdx.x;
    const int blk0 = k1 > k0 ? k0 / a.bs : 0;
    const int nblk = k1 > k0 ? (k1 - 1) / a.bs - blk0 + 1 : 0;
    const int32_t* btab = a.block_table + (size_t)b * a.max_blocks;
    int blk[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int e = tid + i * kW * 64;
        blk[i] = e < nblk ? btab[blk0 + e] : 0;
    }
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_obs);
    uint4 qv[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int e = tid + i * kW * 64;
        const int lane = e & 63, ks = (e >> 6) % KS, t = (e >> 6) / KS;
        const int r = t * 16 + (lane & 15);
        qv[i] = make_uint4(0, 0, 0, 0);
        if (e < NQ && r < a.R) {
            const int h = g * a.G + r / a.w, qi = r % a.w;
            qv[i] = *reinterpret_cast<const uint4*>(qp + (((size_t)b * a.Hq + h) * a.w + qi) * D +
                                                    ks * 32 + (lane >> 4) * 8);
        }
    }
    float rc[RPT];
    if (rowc != nullptr) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = tid + i * kW * 64;
            rc[i] = r < a.R ? rowc[((size_t)b * a.Hkv + g) * a.R + r] : kNegInf;
        }
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int e = tid + i * kW * 64;
        if (e < nblk) {
            unsigned row = kBadRow;
            if ((unsigned)blk[i] < (unsigned)a.num_blocks) row = ((unsigned)blk[i] * a.Hkv + g) * a.bs;
            else bad = true;
            tab[e] = row;
        }
    }
    const unsigned flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int e = tid + i * kW * 64;
        uint4 v = qv[i];
        v.x ^= flip; v.y ^= flip; v.z ^= flip; v.w ^= flip;
        if (e < NQ) qs[e] = v;
    }
    if (rowc != nullptr) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = tid + i * kW * 64;
            if (r < NT * 16) rowc_lds[r] = rc[i];
        }
    }
    return bad;
}

// Load the K rows of one 32-key chunk (keys c0 .. c0+31, each 16 lanes x 16 B) into registers,
// lane (m16, q4) of k-step ks holding row m16, dims ks*32 + q4*8 .. +7 (MFMA operand order).
// c0 is wave-uniform and a multiple of 16, so each 16-key tile's block base is one uniform LDS
// read. Keys outside [k0, k1) or with a bad block load row 0 and are reported as masked.
// (For the passes over many row tiles, loading whole rows per instruction and reordering
// through LDS measured slower: with their score arithmetic in the loop the access pattern is
// not what limits them. The one-tile stored-score pass uses load_k_rows instead.)
template <int D>
__device__ __forceinline__ void load_k(const uint16_t* kp, const unsigned* tab, int bs, int sh,
                                       int blk0, int c0, int k1, int m16, int q4,
                                       uint4 (&kr)[2][D / 32], unsigned (&okm)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const int t0 = c0 + kt * 16;
        unsigned base = kBadRow;
        if (t0 < k1) base = tab[div_bs(t0, bs, sh) - blk0];
        const bool ok = base != kBadRow && t0 + m16 < k1;
        okm[kt] = (unsigned)(__ballot(ok) & 0xffffull);
        const unsigned row = base + (unsigned)(t0 - div_bs(t0, bs, sh) * bs + m16);
        const size_t off = (size_t)(ok ? row : 0u) * D + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            kr[kt][ks] = *reinterpret_cast<const uint4*>(kp + off + ks * 32);   // 64 B per row: plain
    }
}

// The same chunk loaded whole rows per instruction with nontemporal loads: instruction ks of
// tile kt covers the 1 KB of rows ks * RPI .. + RPI - 1 of the tile (RPI = 1024 / (2 D)), lane l
// holding row ks * RPI + l / (D / 8), dims (l % (D / 8)) * 8 .. +7. rows_to_operands turns it
// into load_k's layout. okm as in load_k. The valid rows of a tile are a prefix (the tile lies in
// one block and the range ends at k1), so each tile is read through a buffer resource covering
// just them: masked rows read as zero without a memory access, and one lane offset serves all
// loads.
template <int D>
__device__ __forceinline__ void load_k_rows(const uint16_t* kp, const unsigned* tab, int bs, int sh,
                                            int blk0, int c0, int k1, int lane,
                                            uint4 (&kr)[2][D / 32], unsigned (&okm)[2]) {
    constexpr int kNontemporal = 2;                      // cache-policy bits of the load
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        // No branch around the loads: the table read is clamped into the table (a tile past k1
        // discards what it reads) and the rest are selects on wave-uniform values.
        const int t0 = c0 + kt * 16;
        const int blk = div_bs(t0, bs, sh);
        const unsigned tv = __builtin_amdgcn_readfirstlane(
            tab[min(max(blk - blk0, 0), kSnapTableEntries)]);
        const unsigned base = t0 < k1 ? tv : kBadRow;
        const int n_ok = base != kBadRow ? min(k1 - t0, 16) : 0;
        okm[kt] = n_ok >= 16 ? 0xffffu : (1u << n_ok) - 1u;
        const unsigned row0 = n_ok > 0 ? base + (unsigned)(t0 - blk * bs) : 0u;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(kp + (size_t)row0 * D), (short)0, n_ok * D * 2, kBufferWord3);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + ks * 1024, 0,
                                                                    kNontemporal);
            kr[kt][ks] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
}

// Reorder a chunk from load_k_rows' layout into MFMA operand order through a wave-private LDS
// tile of 16 rows (D / 8 16-byte pieces each), one 16-key tile at a time. Piece p of row j is
// kept in slot p ^ ((j / RP) % (D / 8)), RP = rows per 256 bytes, so that the row-wise writes
// and the operand reads (one piece of each of 16 rows) both meet every bank once per 16 lanes.
// The wave's DS instructions execute in order, so a tile's reads see its writes and the next
// tile's writes come after them.
template <int D>
__device__ __forceinline__ void rows_to_operands(uint4* buf, int lane, uint4 (&kr)[2][D / 32]) {
    constexpr int LPR = D / 8, RPI = 64 / LPR, RP = 128 / D;
    const int m16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        wave_lds_order();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const int j = ks * RPI + lane / LPR, p = lane % LPR;
            buf[j * LPR + (p ^ ((j / RP) % LPR))] = kr[kt][ks];
        }
        wave_lds_order();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const int p = ks * 4 + q4;
            kr[kt][ks] = buf[m16 * LPR + (p ^ ((m16 / RP) % LPR))];
        }
    }
}

// One 16-row tile of the score product for 32 keys (two 16-key tiles), chained over D.
// ROWS_A: queries are the A operand (S = Q . K^T, pass 2); else keys are (S^T = K . Q^T, pass 1).
template <int KS, bool ROWS_A>
__device__ __forceinline__ void score_tile(const uint4 (&qv)[KS], const uint4 (&kr)[2][KS],
                                           f32x4 (&acc)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
            acc[kt] = ROWS_A
                ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(qv[ks]), to_bf16x8(kr[kt][ks]), acc[kt], 0, 0, 0)
                : __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(kr[kt][ks]), to_bf16x8(qv[ks]), acc[kt], 0, 0, 0);
}

// Row constant m + log2 l of observation row r of (b, g) from the pass-1 split partials (log2
// domain): +inf for a row with no keys (it adds nothing), NaN if a split was poisoned. Partials
// are read eight at a time (two passes: the maximum, then the rescaled sum).
__device__ float row_constant(const SnapArgs& a, int b, int g, int r) {
    const float2* pp = reinterpret_cast<const float2*>(a.part1) +
                       (((size_t)b * a.Hkv + g) * a.R + r) * a.nsplit1;
    const int n = a.nsplit1;
    constexpr int kU = 8;
    float M = kNegInf;
    bool nan = false;
    for (int s0 = 0; s0 < n; s0 += kU) {
        float m[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) m[u] = s0 + u < n ? pp[s0 + u].x : kNegInf;
#pragma unroll
        for (int u = 0; u < kU; ++u) { nan |= m[u] != m[u]; M = fmaxf(M, m[u]); }
    }
    float lam = 0.f;
    if (M != kNegInf)
        for (int s0 = 0; s0 < n; s0 += kU) {
            float2 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = s0 + u < n ? pp[s0 + u] : make_float2(kNegInf, 0.f);
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (v[u].x != kNegInf) lam += __builtin_amdgcn_exp2f(v[u].x - M) * v[u].y;
        }
    return nan ? __builtin_nanf("") : (lam > 0.f ? M + __log2f(lam) : __builtin_huge_valf());
}

// Between the passes: -(row constant) of every observation row, once per (sequence, KV head).
__global__ __launch_bounds__(256) void snap_rowconst_kernel(SnapArgs a) {
    const int g = blockIdx.x, b = blockIdx.y;
    for (int r = threadIdx.x; r < a.R; r += 256)
        a.rowc[((size_t)b * a.Hkv + g) * a.R + r] = -row_constant(a, b, g, r);
}

template <int KS>
__device__ __forceinline__ void read_q(const uint4* qs, int t, int lane, uint4 (&qv)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = qs[(t * KS + ks) * 64 + lane];
}

// ---------------------------------------------------------------- pass 1: row statistics
// NT row tiles (16 rows each, rows past R are zero queries whose statistics are not written).
// STORE (one row tile only): also write each row's scaled scores of the candidate keys
// j < P - w to a.xs (NaN for a key whose block id is invalid), for the stored second pass.
// Sixteen row tiles would take 259 registers (one wave per SIMD); bounding them to two
// workgroups per CU costs two spilled registers and runs the pass ~10% faster (256 rows at a
// 100k context: SnapKV select 2.98-3.08 -> 2.71 ms, same selection).
template <int D, int NT, bool STORE>
__global__ __launch_bounds__(kW * 64, NT >= 16 ? 2 : STORE ? 3 : 1) void snap_rowstats_mfma(SnapArgs a) {
    static_assert(!STORE || NT == 1, "stored scores use one row tile");
    constexpr int KS = D / 32;

    constexpr int QS = NT * KS * 64 * 16;                  // queries in MFMA operand order
    constexpr int MS = 2 * kW * NT * 16 * 4;               // per-wave (max, sum), after the loop
    constexpr int TAB = (kSnapTableEntries + 1) * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[(QS > MS ? QS : MS) + TAB];
    uint4* qs = reinterpret_cast<uint4*>(smem);
    float* sm = reinterpret_cast<float*>(smem);             // [kW][NT*16], reuses the queries
    float* sl = sm + kW * NT * 16;
    unsigned* tab = reinterpret_cast<unsigned*>(smem + (QS > MS ? QS : MS));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int k0 = split * a.split_len1;
    const int k1 = (split == a.nsplit1 - 1) ? P : min(k0 + a.split_len1, P);
    const int bs = a.bs, sh = (bs & (bs - 1)) == 0 ? __builtin_ctz(bs) : -1;
    const int blk0 = div_bs(k0, bs, sh);
    // The planner keeps a split within one table; a longer one is refused (poisoned, not read).
    const bool fits = (k1 - k0) <= (kSnapTableEntries - 1) * bs;
    const int kend = fits ? k1 : k0;
    const bool poisoned =
        __syncthreads_or(!fits || stage_prologue<D, NT, kSnapTableEntries + 1>(
                                      a, b, g, k0, kend, tab, qs, nullptr, nullptr)) != 0;

    // The first two chunks are issued after the barrier (they need the block bases). With one
    // row tile the pass has little arithmetic per byte, and there whole-row nontemporal loads
    // reordered through LDS beat operand-order loads (the per-step Top-K search's K read).
    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    constexpr int stride = kW * 32;
    __shared__ uint4 kreorder[STORE ? kW * 16 * (D / 8) : 1];
    uint4* kbuf = kreorder + (STORE ? wid * 16 * (D / 8) : 0);
    auto issue = [&](int c0, uint4 (&kr)[2][KS], unsigned (&okm)[2]) {
        if constexpr (STORE) load_k_rows<D>(kp, tab, bs, sh, blk0, c0, kend, lane, kr, okm);
        else load_k<D>(kp, tab, bs, sh, blk0, c0, kend, m16, q4, kr, okm);
    };
    uint4 kA[2][KS], kB[2][KS];
    unsigned okA[2], okB[2];
    int c = k0 + wid * 32;
    issue(c, kA, okA);
    issue(c + stride, kB, okB);

    // Per lane: online (max, sum) of the scores it holds for row t*16 + m16; the maximum is
    // kept negated (nm = -m) so the exponent is one fma.
    float nm[NT], lr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { nm[t] = -kNegInf; lr[t] = 0.f; }
    const float sc = fabsf(a.scale_log2);
    const int causal_from = P - a.w;            // keys below it are visible to every row
    const int nstore = min(k1, max(causal_from, 0));
    float* xrow = STORE && m16 < a.R
        ? a.xs + (((size_t)b * a.Hkv + g) * a.R + m16) * a.xs_stride : nullptr;

    // Tile t+1's products are issued before tile t's exponentials, so the matrix core and the
    // vector ALU overlap within the wave.
    auto consume = [&](auto full_tag, int c0, const uint4 (&kr)[2][KS], const unsigned (&okm)[2]) {
        constexpr bool FULL = decltype(full_tag)::value;
        uint4 qv[2][KS];
        f32x4 acc[2][2];
        read_q<KS>(qs, 0, lane, qv[0]);
        if (NT > 1) read_q<KS>(qs, 1, lane, qv[1]);
        score_tile<KS, false>(qv[0], kr, acc[0]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // Issue order per tile: the next tile's products, the queries two tiles ahead (into
            // the registers this tile's products no longer need), then this tile's statistics.
            if (t + 1 < NT) score_tile<KS, false>(qv[(t + 1) & 1], kr, acc[(t + 1) & 1]);
            if (t + 2 < NT) read_q<KS>(qs, t + 2, lane, qv[t & 1]);
            const f32x4* s = acc[t & 1];
            if constexpr (STORE) {
                // lane (row m16, group q4) holds keys c0 + 16 kt + 4 q4 + i of its row
                if (xrow != nullptr) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        const int key0 = c0 + kt * 16 + q4 * 4;
                        float x[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            x[i] = ((okm[kt] >> (q4 * 4 + i)) & 1u) ? s[kt][i] * sc : __builtin_nanf("");
                        if (FULL || key0 + 3 < nstore) {
                            *reinterpret_cast<float4*>(xrow + key0) = make_float4(x[0], x[1], x[2], x[3]);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (key0 + i < nstore) xrow[key0 + i] = x[i];
                        }
                    }
                }
            }
            if constexpr (FULL) {
                // Lazy maximum: the reference -nm[t] moves only when a term could overflow the
                // sum, i.e. when some score exceeds it by more than 64 (the tile sum then
                // exceeds 2^64; at the start nm[t] = +inf makes it infinite).
                float p = 0.f;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p += __builtin_amdgcn_exp2f(fmaf(s[kt][i], sc, nm[t]));
                const bool big = !(p <= 0x1p64f);
                if (__ballot(big) != 0ull) {
                    if (big) {
                        // sc >= 0, so the maximum of the raw products scales to the score maximum.
                        const float cm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                               fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
                        const float mnew = fmaxf(-nm[t], cm * sc);
                        lr[t] *= __builtin_amdgcn_exp2f(-nm[t] - mnew);
                        p = 0.f;
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) p += __builtin_amdgcn_exp2f(fmaf(s[kt][i], sc, -mnew));
                        nm[t] = -mnew;
                    }
                }
                lr[t] += p;
            } else {
                const int lim = causal_from + ((t * 16 + m16) % a.w);   // causal bound of the row
                float x[8];
                float cm = kNegInf;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = kt * 16 + q4 * 4 + i;
                        const bool ok = ((okm[kt] >> (q4 * 4 + i)) & 1u) && (c0 + key <= lim);
                        x[kt * 4 + i] = ok ? s[kt][i] * sc : kNegInf;
                        cm = fmaxf(cm, x[kt * 4 + i]);
                    }
                const float mold = -nm[t];
                const float mnew = fmaxf(mold, cm);
                const float ms = mnew == kNegInf ? 0.f : mnew;    // no key yet: every term is 0
                float sum = lr[t] * __builtin_amdgcn_exp2f(mold - ms);
#pragma unroll
                for (int j = 0; j < 8; ++j) sum += __builtin_amdgcn_exp2f(x[j] - ms);
                lr[t] = sum;
                nm[t] = -mnew;
            }
            __builtin_amdgcn_sched_barrier(0);      // keep the per-tile issue order
        }
    };
    auto step = [&](int c0, uint4 (&kr)[2][KS], const unsigned (&okm)[2]) {
        if constexpr (STORE) rows_to_operands<D>(kbuf, lane, kr);
        // Uniform: every key of the chunk is valid and visible to every row.
        if ((okm[0] & okm[1]) == 0xffffu && c0 + 31 < causal_from)
            consume(std::true_type{}, c0, kr, okm);
        else
            consume(std::false_type{}, c0, kr, okm);
    };

    // Two chunks in flight per wave: consume one, then reissue its registers two chunks ahead.
    for (; c < kend; c += 2 * stride) {
        step(c, kA, okA);
        issue(c + 2 * stride, kA, okA);
        if (c + stride >= kend) break;
        step(c + stride, kB, okB);
        issue(c + 3 * stride, kB, okB);
    }

    // Merge the 4 lane groups (xor 16, 32) and then the waves, per row.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float mr = -nm[t];
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            const float m2 = __shfl_xor(mr, o), l2 = __shfl_xor(lr[t], o);
            const float M = fmaxf(mr, m2);
            const float Ms = M == kNegInf ? 0.f : M;
            lr[t] = lr[t] * __builtin_amdgcn_exp2f(mr - Ms) + l2 * __builtin_amdgcn_exp2f(m2 - Ms);
            mr = M;
        }
        nm[t] = -mr;
    }
    __syncthreads();                                        // every wave is done with the queries
#pragma unroll
    for (int t = 0; t < NT; ++t)
        if (q4 == 0) { sm[wid * NT * 16 + t * 16 + m16] = -nm[t]; sl[wid * NT * 16 + t * 16 + m16] = lr[t]; }
    __syncthreads();
    for (int r = tid; r < a.R; r += kW * 64) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kW; ++w) M = fmaxf(M, sm[w * NT * 16 + r]);
        float L = 0.f;
        if (M != kNegInf)
#pragma unroll
            for (int w = 0; w < kW; ++w) L += sl[w * NT * 16 + r] * __builtin_amdgcn_exp2f(sm[w * NT * 16 + r] - M);
        float* pp = a.part1 + ((((size_t)b * a.Hkv + g) * a.R + r) * a.nsplit1 + split) * 2;
        pp[0] = poisoned ? __builtin_nanf("") : M;
        pp[1] = poisoned ? __builtin_nanf("") : L;
    }
}

// ---------------------------------------------------------------- pass 2: column scores
template <int D, int NT>
__global__ __launch_bounds__(kW * 64) void snap_colscore_mfma(SnapArgs a) {
    constexpr int KS = D / 32;

    constexpr int QS = NT * KS * 64 * 16;
    constexpr int TAB = (kSnapColKeys / 16 + 2) * 4;        // block bases of kSnapColKeys keys
    __shared__ __attribute__((aligned(16))) unsigned char smem[QS + TAB];
    __shared__ __attribute__((aligned(16))) float rowc[NT * 16];
    uint4* qs = reinterpret_cast<uint4*>(smem);
    unsigned* tab = reinterpret_cast<unsigned*>(smem + QS);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int n = max(P - a.w, 0);
    const int k0 = tile * kSnapColKeys;
    if (k0 >= n) return;
    const int k1 = min(k0 + kSnapColKeys, n);
    const int bs = a.bs, sh = (bs & (bs - 1)) == 0 ? __builtin_ctz(bs) : -1;
    const int blk0 = div_bs(k0, bs, sh);
    // A operand of S = Q . K^T: lane supplies row m16 of the tile and dims q4*8.. of k-step ks,
    // which is exactly the operand-order staging used for the B operand of pass 1. The row
    // constants are negated (one fma per term).
    const bool poisoned =
        __syncthreads_or(stage_prologue<D, NT, kSnapColKeys / 16 + 2>(a, b, g, k0, k1, tab, qs,
                                                                       a.rowc, rowc)) != 0;

    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    constexpr int stride = kW * 32;
    uint4 kA[2][KS], kB[2][KS];
    unsigned okA[2], okB[2];
    int c = k0 + wid * 32;
    load_k<D>(kp, tab, bs, sh, blk0, c, k1, m16, q4, kA, okA);
    load_k<D>(kp, tab, bs, sh, blk0, c + stride, k1, m16, q4, kB, okB);

    float* dst = a.scores + ((size_t)b * a.Hkv + g) * a.n_stride;
    const float sc = fabsf(a.scale_log2);

    auto consume = [&](int c0, const uint4 (&kr)[2][KS], const unsigned (&okm)[2]) {
        float col[2] = {0.f, 0.f};
        uint4 qv[2][KS];
        f32x4 acc[2][2];
        read_q<KS>(qs, 0, lane, qv[0]);
        if (NT > 1) read_q<KS>(qs, 1, lane, qv[1]);
        score_tile<KS, true>(qv[0], kr, acc[0]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t + 1 < NT) score_tile<KS, true>(qv[(t + 1) & 1], kr, acc[(t + 1) & 1]);
            if (t + 2 < NT) read_q<KS>(qs, t + 2, lane, qv[t & 1]);
            const f32x4* cur = acc[t & 1];
            const float4 rc = *reinterpret_cast<const float4*>(&rowc[t * 16 + q4 * 4]);   // -row constant
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const f32x4& s = cur[kt];
                col[kt] += __builtin_amdgcn_exp2f(fmaf(s[0], sc, rc.x)) +
                           __builtin_amdgcn_exp2f(fmaf(s[1], sc, rc.y)) +
                           __builtin_amdgcn_exp2f(fmaf(s[2], sc, rc.z)) +
                           __builtin_amdgcn_exp2f(fmaf(s[3], sc, rc.w));
            }
            __builtin_amdgcn_sched_barrier(0);      // keep the per-tile issue order
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

    for (; c < k1; c += 2 * stride) {
        consume(c, kA, okA);
        load_k<D>(kp, tab, bs, sh, blk0, c + 2 * stride, k1, m16, q4, kA, okA);
        if (c + stride >= k1) break;
        consume(c + stride, kB, okB);
        load_k<D>(kp, tab, bs, sh, blk0, c + 3 * stride, k1, m16, q4, kB, okB);
    }
}

// ---------------------------------------------------------------- pass 2 from stored scores
// c[j] = sum_r 2^(x[r][j] - m_r - log2 l_r) over the R <= 16 stored rows; 4 keys per thread,
// one 16-byte load per row.
constexpr int kStoredKeys = kW * 64 * 4;

__global__ __launch_bounds__(kW * 64) void snap_colscore_stored(SnapArgs a) {
    __shared__ float rowc[16];
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int P = max(min(a.prompt_lens[b], a.max_kv_len), 0);
    const int n = max(P - a.w, 0);
    const int k0 = tile * kStoredKeys;
    if (k0 >= n) return;
    if (tid < a.R) rowc[tid] = a.rowc[((size_t)b * a.Hkv + g) * a.R + tid];
    __syncthreads();
    const int j = k0 + 4 * tid;
    if (j >= n) return;
    const float* xb = a.xs + ((size_t)b * a.Hkv + g) * a.R * a.xs_stride + j;
    float c[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < a.R; ++r) {
        const float4 x = load_stream_f4(xb + (size_t)r * a.xs_stride);
        const float rc = rowc[r];
        c[0] += __builtin_amdgcn_exp2f(x.x + rc);
        c[1] += __builtin_amdgcn_exp2f(x.y + rc);
        c[2] += __builtin_amdgcn_exp2f(x.z + rc);
        c[3] += __builtin_amdgcn_exp2f(x.w + rc);
    }
    float* dst = a.scores + ((size_t)b * a.Hkv + g) * a.n_stride + j;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (j + i < n) dst[i] = c[i];
}

template <int D, int NT>
hipError_t launch_passes(const SnapArgs& a, hipStream_t s) {
    if constexpr (NT == 1) {
        if (a.xs != nullptr) {
            snap_rowstats_mfma<D, 1, true><<<dim3(a.nsplit1, a.Hkv, a.B), kW * 64, 0, s>>>(a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || a.n_stride == 0) return e;
            snap_rowconst_kernel<<<dim3(a.Hkv, a.B), 256, 0, s>>>(a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const dim3 grid((a.n_stride + kStoredKeys - 1) / kStoredKeys, a.Hkv, a.B);
            snap_colscore_stored<<<grid, kW * 64, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    snap_rowstats_mfma<D, NT, false><<<dim3(a.nsplit1, a.Hkv, a.B), kW * 64, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_stride == 0) return e;
    snap_rowconst_kernel<<<dim3(a.Hkv, a.B), 256, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((a.n_stride + kSnapColKeys - 1) / kSnapColKeys, a.Hkv, a.B);
    snap_colscore_mfma<D, NT><<<grid, kW * 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SnapArgs& a, hipStream_t s) {
    // One row tile up to 16 rows, else row tiles rounded up to an even count (R <= 256 rows:
    // at most 16 tiles).
    if (a.R <= 16) return launch_passes<D, 1>(a, s);
    switch ((((a.R + 15) / 16) + 1) / 2) {
        case 1: return launch_passes<D, 2>(a, s);
        case 2: return launch_passes<D, 4>(a, s);
        case 3: return launch_passes<D, 6>(a, s);
        case 4: return launch_passes<D, 8>(a, s);
        case 5: return launch_passes<D, 10>(a, s);
        case 6: return launch_passes<D, 12>(a, s);
        case 7: return launch_passes<D, 14>(a, s);
        case 8: return launch_passes<D, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_snapkv_mfma_passes(const SnapArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace kvss
