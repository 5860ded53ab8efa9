// Speculative acceptance (MagicDec Section 3.1: the speculative-decoding rule of Leviathan et
// al., whose expected yield is Eq. (1); Section 5.1: greedy decoding in the experiments).
//
// Kernels, in launch order:
//   stats    grid (slice, row, sequence): each workgroup streams one slice of one logit row
//            (target rows 0..gamma, draft rows 0..gamma-1) once with 16-byte loads and writes a
//            partial (a reference r, the sum of 2^(z log2(e) / temp - r), max z, its lowest
//            index); the reference moves only when a term would pass 2^64, so the common block
//            of 4 tokens costs four fma + exp2 and no data-dependent branch. When sampling,
//            the slices of target row gamma also run the race for the token emitted after full
//            acceptance: p_gamma needs no statistics, its race key being ln E - z / temp;
//   decide   one wave per sequence, a lane per logit row: merges each row's partials into its
//            statistics, runs the gamma accept tests in parallel lanes (greedy argmax match, or
//            u_i < p_i(x_i) / q_i(x_i) with Philox uniforms), takes the first failing lane, and
//            writes the accepted prefix and the count; after full acceptance it also emits the
//            statistics pass's race winner, else it records the emitting position and the log
//            normalisers of its row pair for the race;
//   race     (sampling, after a rejection) grid (slice, sequence): exponential race
//            argmin_x -log(u'_x) / w(x), w = max(0, p - q), over one slice of the emitting row
//            pair, branch-free, several 16-byte loads in flight per thread;
//   finalize (sampling, after a rejection) one wave per sequence: the winning token of the
//            slices (the race over p itself if w vanished everywhere).
// (A completion counter that let the race's last workgroup finalize measured slower than this
// separate launch: the device-scope fences it needs in every workgroup cost more.)
// Argmax: the lowest index of the maximum over the row's non-NaN entries; a row with no such
// entry has argmax -1. The streaming passes track only entries above -inf; a row without one is
// rescanned by the decide kernel (its argmax is then its first non-NaN entry).

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kStatThreads = 256;
constexpr int kRaceThreads = 256;
#ifndef KVSS_STAT_TOKENS
#define KVSS_STAT_TOKENS 16384
#endif
#ifndef KVSS_RACE_TOKENS
#define KVSS_RACE_TOKENS 2048
#endif
constexpr int kStatTokens = KVSS_STAT_TOKENS;   // logits per statistics workgroup
constexpr int kRaceTokens = KVSS_RACE_TOKENS;   // logits per race workgroup (small: the race is
                                                // Philox-bound, and short workgroups overlap it
                                                // with the loads of others)
constexpr uint32_t kRaceStream = 1;     // Philox stream of the race uniforms

struct Part {          // per (sequence, row, slice)
    float m2;          // reference of the sum in log2 units (<= max of z * log2(e) / t)
    float s;           // sum of 2^(z * log2(e) / t - m2)
    float zmax;        // max z and its lowest index
    int imax;
};

struct RaceKey {
    float key;
    int x;
};

struct Decision {      // per sequence
    int pos;           // emitting position (= number accepted)
    float ct;          // emitting target row: log2 of its softmax normaliser, (max z / t) log2(e)
                       // + log2(sum of exp), so p(x) = 2^(z(x) log2(e) / t - ct)
    float cd;          // the same for the emitting draft row after a rejection (0 otherwise)
    int pad;
};

constexpr int kNoArgmax = 0x7fffffff;   // no non-NaN entry seen

// (reference, sum) pairs in the log2 domain
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == kNegInf) { m = kNegInf; s = 0.f; return; }
    s = s * __builtin_amdgcn_exp2f(m - M) + s2 * __builtin_amdgcn_exp2f(m2 - M);
    m = M;
}

__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ __forceinline__ void race_merge(RaceKey& a, RaceKey b) {
    if (b.key < a.key || (b.key == a.key && b.x < a.x)) a = b;
}

__device__ __forceinline__ const float* row_ptr(const AcceptArgs& a, int b, int r) {
    const int gamma = a.gamma;
    return (r <= gamma) ? a.target + ((size_t)b * (gamma + 1) + r) * a.V
                        : a.draft + ((size_t)b * gamma + (r - gamma - 1)) * a.V;
}

// Statistics of one logit row from its slice partials: m = max of z / t (exactly (max z) / t:
// rounding is monotone), s = sum of exp(z / t - m), and the argmax.
// The partials are read eight at a time (all eight loads in flight), then merged in slice
// order.
__device__ __forceinline__ void row_stats(const Part* p, int nslice, float it, bool greedy,
                                          float& m, float& s, float& best, int& bi) {
    constexpr int kBatch = 8;
    float m2 = kNegInf, s2 = 0.f;
    best = kNegInf;
    bi = kNoArgmax;
    for (int k0 = 0; k0 < nslice; k0 += kBatch) {
        Part q[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            q[u] = k0 + u < nslice ? p[k0 + u] : Part{kNegInf, 0.f, kNegInf, kNoArgmax};
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (!greedy) ms_merge(m2, s2, q[u].m2, q[u].s);
            am_merge(best, bi, q[u].zmax, q[u].imax);
        }
    }
    m = best * it;
    s = 0.f;
    if (!greedy && best != kNegInf) s = s2 * __builtin_amdgcn_exp2f(m2 - best * (it * kLog2e));
}

// Lowest index of a non-NaN entry of row z[0, V), or -1; the whole wave scans (used only for a
// row in which no entry exceeds -inf, whose argmax is then its first -inf entry).
__device__ int first_non_nan(const float* z, int V, int lane) {
    int found = 0x7fffffff;
    for (int x0 = 0; x0 < V; x0 += 8 * 64) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = x0 + u * 64 + lane < V ? z[x0 + u * 64 + lane] : __builtin_nanf("");
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (v[u] == v[u]) found = min(found, x0 + u * 64 + lane);
        for (int o = 32; o > 0; o >>= 1) found = min(found, __shfl_xor(found, o));
        if (found != 0x7fffffff) return found;
    }
    return -1;
}

// Statistics-free race key of token x over p = softmax(z / t): log2(-log2 u_x) - z_x log2(e) / t
// orders tokens as ln E_x - z_x / t does (E_x = -ln u_x), i.e. as E_x / p(x).
__device__ __forceinline__ float p_race_key(uint32_t word, float z, float c) {
    const float lu = __builtin_amdgcn_logf(philox_uniform(word));       // log2 u < 0
    return fmaf(-z, c, __builtin_amdgcn_logf(-lu));
}

template <bool GREEDY>
__global__ __launch_bounds__(kStatThreads) void accept_stats_kernel(AcceptArgs a, Part* parts,
                                                                    int nslice, RaceKey* bonus) {
    __shared__ Part sp[kStatThreads / 64];
    __shared__ RaceKey sb[kStatThreads / 64];
    const int slice = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int rows = gridDim.y;
    // target row gamma: also the race over p_gamma for the token after full acceptance
    const bool race_p = !GREEDY && r == a.gamma;
    RaceKey bk{__builtin_huge_valf(), 0x7fffffff};
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    const uint32_t w1 = ((uint32_t)kRaceStream << 16) | (uint32_t)a.gamma;
    const float* z = row_ptr(a, b, r);
    // slice bounds in float4 units (16-byte aligned rows with V % 4 == 0) or elements
    const bool vec = (a.V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0;
    const int units = vec ? a.V / 4 : a.V;
    const int per = (units + nslice - 1) / nslice;
    const int u0 = slice * per, u1 = min(units, u0 + per);
    const float c = a.inv_temp * kLog2e;
    float m = kNegInf, s = 0.f, best = kNegInf;
    int bi = kNoArgmax;
    // Block of n <= 4 tokens x0 .. x0 + n - 1. The sum keeps a lazy reference m: a block's terms
    // 2^(z c - m) are added as they are unless their sum leaves [0, 2^64] (a score more than 64
    // above m, or the first block with m = -inf); only then does m move to the block's max.
    auto visit = [&](const float (&v)[4], int x0, int n) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n && v[e] > best) { best = v[e]; bi = x0 + e; }    // increasing x per thread
        if (race_p) {
            // uniforms: word x % 4 of Philox block x / 4 at (x / 4, stream << 16 | gamma, b, offset)
            uint32_t w0 = (uint32_t)(x0 >> 2), ww1 = w1, w2 = (uint32_t)b, w3 = (uint32_t)a.offset;
            philox4x32_10(w0, ww1, w2, w3, k0, k1);
            const uint32_t w[4] = {w0, ww1, w2, w3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = x0 + e;
                if (e < n) {
                    const float key = p_race_key(w[x & 3], v[e], c);
                    if (key < bk.key) bk = RaceKey{key, x};
                }
            }
        }
        if constexpr (!GREEDY) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < n) t += __builtin_amdgcn_exp2f(fmaf(v[e], c, -m));
            if (!(t <= 0x1p64f)) {
                float bm = kNegInf;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < n) bm = fmaxf(bm, v[e] * c);
                const float mnew = fmaxf(m, bm);
                const float ms = mnew == kNegInf ? 0.f : mnew;
                s *= __builtin_amdgcn_exp2f(m - ms);
                t = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < n) t += __builtin_amdgcn_exp2f(fmaf(v[e], c, -ms));
                m = mnew;
            }
            s += t;
        }
    };
    if (vec) {
        const float4* z4 = reinterpret_cast<const float4*>(z);
        int j = u0 + tid;
        for (; j + 3 * kStatThreads < u1; j += 4 * kStatThreads) {
            float4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = load_stream_f4(z4 + j + q * kStatThreads);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
                visit(w, 4 * (j + q * kStatThreads), 4);
            }
        }
        for (; j < u1; j += kStatThreads) {
            const float4 v = load_stream_f4(z4 + j);
            const float w[4] = {v.x, v.y, v.z, v.w};
            visit(w, 4 * j, 4);
        }
    } else {
        for (int j = u0 + tid; j < u1; j += kStatThreads) {
            const float w[4] = {z[j], 0.f, 0.f, 0.f};
            visit(w, j, 1);
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o), b2 = __shfl_xor(best, o);
        const int i2 = __shfl_xor(bi, o);
        if constexpr (!GREEDY) ms_merge(m, s, m2, s2);
        am_merge(best, bi, b2, i2);
        if (race_p) race_merge(bk, {__shfl_xor(bk.key, o), __shfl_xor(bk.x, o)});
    }
    const int lane = tid & 63, wid = tid >> 6;
    if (lane == 0) { sp[wid] = Part{m, s, best, bi}; sb[wid] = bk; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kStatThreads / 64; ++w) {
            if constexpr (!GREEDY) ms_merge(m, s, sp[w].m2, sp[w].s);
            am_merge(best, bi, sp[w].zmax, sp[w].imax);
            race_merge(bk, sb[w]);
        }
        parts[(((size_t)b * rows) + r) * nslice + slice] = Part{m, s, best, bi};
        if (race_p) bonus[(size_t)b * nslice + slice] = bk;
    }
}

// The acceptance walk of sequence b by one wave, a lane per logit row (rows = gamma + 1 target
// rows, then, when sampling, gamma draft rows): each lane merges its row's slice partials; lane
// i < gamma runs accept test i; the first failing lane is the emitting position. With `write`,
// the accepted prefix, the count and the row statistics are written (the emitted token's slot
// gets its greedy argmax, or -1 for the race to fill). Returns the decision in every lane.
// Lanes exchange values by shuffles only, so any one wave of a workgroup may run it.
__device__ Decision decide_wave(const AcceptArgs& a, const Part* parts, int nslice, int rows,
                                int b, int lane, bool write) {
    const int gamma = a.gamma, V = a.V;
    const bool greedy = a.inv_temp == 0.f;
    // this lane's draft token (lanes i < gamma: position i; draft rows gamma+1+i: position i)
    const int ti = lane < gamma ? lane : lane - gamma - 1;
    const bool has_tok = (lane < gamma) || (!greedy && lane > gamma && lane < rows);
    const int x = has_tok ? a.tokens[(size_t)b * gamma + ti] : -1;
    float m = 0.f, s = 0.f, zx = 0.f;
    int bi = kNoArgmax;
    if (lane < rows) {
        float best;
        row_stats(parts + ((size_t)b * rows + lane) * nslice, nslice, a.inv_temp, greedy, m, s, best, bi);
        if (!greedy && lane != gamma) zx = (x >= 0 && x < V) ? row_ptr(a, b, lane)[x] * a.inv_temp : kNegInf;
    }
    // A row in which no entry exceeds -inf: its argmax is its first non-NaN entry (-1 if none).
    for (unsigned long long need = __ballot(lane < rows && bi == kNoArgmax); need != 0ull;
         need &= need - 1) {
        const int r = __ffsll((long long)need) - 1;
        const int arg = first_non_nan(row_ptr(a, b, r), V, lane);
        if (lane == r) bi = arg;
    }
    const int arg = bi;
    if (write && a.stats != nullptr) {
        if (lane < rows) {
            float* o = a.stats + ((size_t)b * (2 * gamma + 1) + lane) * 4;
            o[0] = greedy ? 0.f : m;
            o[1] = greedy ? 0.f : s;
            o[2] = zx;
            o[3] = (float)arg;
        }
        // greedy reads no draft rows: their statistics rows are written as zeros
        if (greedy)
            for (int r = rows + lane; r < 2 * gamma + 1; r += 64) {
                float* o = a.stats + ((size_t)b * (2 * gamma + 1) + r) * 4;
                o[0] = 0.f; o[1] = 0.f; o[2] = 0.f; o[3] = 0.f;
            }
    }
    // the draft row of position i is row gamma + 1 + i (rows <= 63: gamma <= 31)
    const int dl = (gamma + 1 + lane) & 63;
    const float md = __shfl(m, dl), sd = __shfl(s, dl), zd = __shfl(zx, dl);
    bool ok = true;
    if (lane < gamma) {
        if (greedy) {
            ok = x >= 0 && arg == x;
        } else {
            // p(x) / q(x) as one exp2 of a difference of logs: at a low temperature p(x) and
            // q(x) alone can underflow float while their ratio is ordinary.
            const float lp = (zx - m) * kLog2e - __log2f(s);
            const float lq = (zd - md) * kLog2e - __log2f(sd);
            uint32_t c0 = 0, c1 = (uint32_t)lane, c2 = (uint32_t)b, c3 = (uint32_t)a.offset;
            philox4x32_10(c0, c1, c2, c3, (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
            ok = (x >= 0 && x < V) && philox_uniform(c0) < __builtin_amdgcn_exp2f(lp - lq);
        }
    }
    const unsigned long long fail = __ballot(!ok);
    const int n = fail ? __ffsll((long long)fail) - 1 : gamma;
    if (write) {
        int32_t* out = a.out_tokens + (size_t)b * (gamma + 1);
        if (lane < n) out[lane] = x;
        else if (lane == n) out[lane] = greedy ? arg : -1;     // sampling: the race fills it
        else if (lane <= gamma) out[lane] = -1;
        if (lane == 0) a.out_num[b] = n;
    }
    Decision r{};
    r.pos = n;
    const float mn = __shfl(m, n), sn = __shfl(s, n);
    const float mdn = __shfl(m, (gamma + 1 + n) & 63), sdn = __shfl(s, (gamma + 1 + n) & 63);
    if (!greedy) {
        r.ct = fmaf(mn, kLog2e, __log2f(sn));
        if (n < gamma) r.cd = fmaf(mdn, kLog2e, __log2f(sdn));
    }
    return r;
}

// One wave per sequence: the acceptance walk. When sampling, it records the decision for the race
// kernel and, after full acceptance, emits the statistics pass's race winner over p_gamma.
__global__ __launch_bounds__(64) void accept_decide_kernel(AcceptArgs a, const Part* parts,
                                                           int nslice, int rows,
                                                           const RaceKey* bonus, Decision* dec) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const Decision d = decide_wave(a, parts, nslice, rows, b, lane, true);
    if (a.inv_temp == 0.f) return;
    if (lane == 0) dec[b] = d;
    if (d.pos == a.gamma) {
        RaceKey bk{__builtin_huge_valf(), 0x7fffffff};
        for (int k = lane; k < nslice; k += 64) race_merge(bk, bonus[(size_t)b * nslice + k]);
        for (int o = 32; o > 0; o >>= 1) race_merge(bk, {__shfl_xor(bk.key, o), __shfl_xor(bk.x, o)});
        if (lane == 0) a.out_tokens[(size_t)b * (a.gamma + 1) + a.gamma] = bk.x;
    }
}

// Sampling after a rejection: the race over one slice of the emitting row pair.
__global__ __launch_bounds__(kRaceThreads) void accept_race_kernel(AcceptArgs a, const Decision* dec,
                                                                   RaceKey* race, int nrace) {
    __shared__ RaceKey sr[kRaceThreads / 64];
    const int slice = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int gamma = a.gamma, V = a.V;
    const float c1 = a.inv_temp * kLog2e;
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    const uint32_t off = (uint32_t)a.offset;
    const Decision d = dec[b];
    const int pos = d.pos;
    if (pos == gamma) return;                    // full acceptance: emitted by the decide kernel
    int32_t* out = a.out_tokens + (size_t)b * (gamma + 1) + pos;
    // After a rejection at pos: w(x) = max(0, p(x) - q(x)), p(x) = 2^(z(x) c1 - ct) and q alike,
    // one FMA and one v_exp each.
    const float* zt = a.target + ((size_t)b * (gamma + 1) + pos) * V;
    const float* zd = a.draft + ((size_t)b * gamma + pos) * V;
    const float ct = d.ct, cd = d.cd;
    const uint32_t w1 = ((uint32_t)kRaceStream << 16) | (uint32_t)pos;
    const int nblk = (V + 3) / 4;
    const int per = (nblk + nrace - 1) / nrace;
    const int j0 = slice * per, j1 = min(nblk, j0 + per);
    RaceKey br{__builtin_huge_valf(), 0x7fffffff};
    // rows are read as one 16-byte load per block of 4 tokens when they are 16-byte aligned
    const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(zt) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(zd) & 15) == 0;
    // One block of 4 tokens: its Philox words, then each token's race key E_x / w(x) (with E_x
    // in log2 units: -log2 u_x, a common factor), branch-free; a thread visits its tokens in
    // increasing order, so a strict compare keeps the lowest token on ties.
    auto block = [&](int j, const float (&vt)[4], const float (&vd)[4]) {
        uint32_t w0 = (uint32_t)j, ww1 = w1, w2 = (uint32_t)b, w3 = off;
        philox4x32_10(w0, ww1, w2, w3, k0, k1);
        const uint32_t w[4] = {w0, ww1, w2, w3};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = 4 * j + e;
            const float E = -__builtin_amdgcn_logf(philox_uniform(w[e]));
            const float rr = __builtin_amdgcn_exp2f(fmaf(vt[e], c1, -ct)) -
                             __builtin_amdgcn_exp2f(fmaf(vd[e], c1, -cd));
            const float key = rr > 0.f && x < V ? E * __builtin_amdgcn_rcpf(rr) : __builtin_huge_valf();
            const bool better = key < br.key;
            br.key = better ? key : br.key;
            br.x = better ? x : br.x;
        }
    };
    constexpr int kBatch = 4;                   // 16-byte loads in flight per thread and row
    int j = j0 + tid;
    if (vec) {
        const float4* t4p = reinterpret_cast<const float4*>(zt);
        const float4* d4p = reinterpret_cast<const float4*>(zd);
        for (; j + (kBatch - 1) * kRaceThreads < j1; j += kBatch * kRaceThreads) {
            float vt[kBatch][4], vd[kBatch][4];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const float4 t4 = load_stream_f4(t4p + j + q * kRaceThreads);
                const float4 d4 = load_stream_f4(d4p + j + q * kRaceThreads);
                vt[q][0] = t4.x; vt[q][1] = t4.y; vt[q][2] = t4.z; vt[q][3] = t4.w;
                vd[q][0] = d4.x; vd[q][1] = d4.y; vd[q][2] = d4.z; vd[q][3] = d4.w;
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) block(j + q * kRaceThreads, vt[q], vd[q]);
        }
    }
    for (; j < j1; j += kRaceThreads) {
        float vt[4], vd[4];
        if (vec) {
            const float4 t4 = load_stream_f4(reinterpret_cast<const float4*>(zt) + j);
            const float4 d4 = load_stream_f4(reinterpret_cast<const float4*>(zd) + j);
            vt[0] = t4.x; vt[1] = t4.y; vt[2] = t4.z; vt[3] = t4.w;
            vd[0] = d4.x; vd[1] = d4.y; vd[2] = d4.z; vd[3] = d4.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = min(4 * j + e, V - 1);
                vt[e] = zt[x];
                vd[e] = zd[x];
            }
        }
        block(j, vt, vd);
    }
    for (int o = 32; o > 0; o >>= 1) race_merge(br, {__shfl_xor(br.key, o), __shfl_xor(br.x, o)});
    if (lane == 0) sr[wid] = br;
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kRaceThreads / 64; ++w) race_merge(br, sr[w]);
        race[(size_t)b * nrace + slice] = br;
    }
}

// Sampling after a rejection: one wave per sequence merges the slices' keys (a slice per lane)
// and writes the token; if max(0, p - q) vanished everywhere it runs the race over p itself.
__global__ __launch_bounds__(64) void accept_finalize_kernel(AcceptArgs a, const Decision* dec,
                                                             const RaceKey* race, int nrace) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const Decision d = dec[b];
    const int pos = d.pos;
    if (pos == a.gamma) return;                  // full acceptance: emitted by the decide kernel
    RaceKey br{__builtin_huge_valf(), 0x7fffffff};
    for (int k = lane; k < nrace; k += 64) race_merge(br, race[(size_t)b * nrace + k]);
    for (int o = 32; o > 0; o >>= 1) race_merge(br, {__shfl_xor(br.key, o), __shfl_xor(br.x, o)});
    if (br.x == 0x7fffffff) {
        const float* zt = a.target + ((size_t)b * (a.gamma + 1) + pos) * a.V;
        const float c1 = a.inv_temp * kLog2e;
        for (int j = lane; 4 * j < a.V; j += 64) {
            uint32_t w0 = (uint32_t)j, w1 = ((uint32_t)kRaceStream << 16) | (uint32_t)pos,
                     w2 = (uint32_t)b, w3 = (uint32_t)a.offset;
            philox4x32_10(w0, w1, w2, w3, (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
            const uint32_t w[4] = {w0, w1, w2, w3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = 4 * j + e;
                if (x < a.V) {
                    const float key = p_race_key(w[e], zt[x], c1);
                    if (key < br.key) br = RaceKey{key, x};
                }
            }
        }
        for (int o = 32; o > 0; o >>= 1) race_merge(br, {__shfl_xor(br.key, o), __shfl_xor(br.x, o)});
    }
    if (lane == 0) a.out_tokens[(size_t)b * (a.gamma + 1) + pos] = br.x;
}

}  // namespace

AcceptPlan accept_plan(int B, int gamma, int V) {
    AcceptPlan p;
    p.nslice = V >= 8192 ? (V + kStatTokens - 1) / kStatTokens : 1;
    p.nrace = V >= 8192 ? (V + kRaceTokens - 1) / kRaceTokens : 1;
    const size_t rows = (size_t)B * (2 * gamma + 1);
    p.parts_bytes = (rows * p.nslice * sizeof(Part) + 255) / 256 * 256;
    p.bonus_bytes = ((size_t)B * p.nslice * sizeof(RaceKey) + 255) / 256 * 256;
    p.race_bytes = ((size_t)B * p.nrace * sizeof(RaceKey) + 255) / 256 * 256;
    p.dec_bytes = ((size_t)B * sizeof(Decision) + 255) / 256 * 256;
    return p;
}

hipError_t launch_accept(const AcceptArgs& a, void* ws, hipStream_t s) {
    const bool greedy = a.inv_temp == 0.f;
    const int rows = greedy ? a.gamma + 1 : 2 * a.gamma + 1;
    const AcceptPlan p = accept_plan(a.B, a.gamma, a.V);
    char* w = static_cast<char*>(ws);
    Part* parts = reinterpret_cast<Part*>(w);
    RaceKey* bonus = reinterpret_cast<RaceKey*>(w + p.parts_bytes);
    RaceKey* race = reinterpret_cast<RaceKey*>(w + p.parts_bytes + p.bonus_bytes);
    Decision* dec = reinterpret_cast<Decision*>(w + p.parts_bytes + p.bonus_bytes + p.race_bytes);
    const dim3 sgrid(p.nslice, rows, a.B);
    if (greedy) accept_stats_kernel<true><<<sgrid, kStatThreads, 0, s>>>(a, parts, p.nslice, bonus);
    else accept_stats_kernel<false><<<sgrid, kStatThreads, 0, s>>>(a, parts, p.nslice, bonus);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    accept_decide_kernel<<<a.B, 64, 0, s>>>(a, parts, p.nslice, rows, bonus, dec);
    if ((e = hipGetLastError()) != hipSuccess || greedy) return e;
    accept_race_kernel<<<dim3(p.nrace, a.B), kRaceThreads, 0, s>>>(a, dec, race, p.nrace);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    accept_finalize_kernel<<<a.B, 64, 0, s>>>(a, dec, race, p.nrace);
    return hipGetLastError();
}

}  // namespace kvss
