// Speculative acceptance (MagicDec Section 3.1: the speculative-decoding rule of Leviathan et
// al., whose expected yield is Eq. (1); Section 5.1: greedy decoding in the experiments).
//
// Two kernels:
//   stats  : one workgroup per logit row (target rows 0..gamma, draft rows 0..gamma-1) streams
//            the vocabulary once with 16-byte loads and reduces max(z/temp), sum exp(z/temp -
//            max), the argmax (lowest id on ties) and z/temp at the row's draft token;
//   decide : one workgroup per sequence. Lane 0 walks the gamma accept tests (greedy argmax
//            match, or u_i < p_i(x_i) / q_i(x_i) with Philox uniforms); the whole workgroup
//            then runs the exponential race argmin_x -log(u'_x) / w(x) over the emitting row
//            (w = max(0, p - q) after a rejection, p after full acceptance), re-reading only
//            that row pair.

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kStatThreads = 256;
constexpr int kRaceThreads = 1024;

struct MaxSum {
    float m, s;
};

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
    const float M = fmaxf(a.m, b.m);
    if (M == kNegInf) return {kNegInf, 0.f};
    return {M, a.s * __expf(a.m - M) + b.s * __expf(b.m - M)};
}

// argmax with lowest-index tie-break
__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

template <bool GREEDY>
__global__ __launch_bounds__(kStatThreads) void accept_stats_kernel(AcceptArgs a) {
    __shared__ float sm[kStatThreads / 64], ss[kStatThreads / 64], sv[kStatThreads / 64];
    __shared__ int si[kStatThreads / 64];
    const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int gamma = a.gamma, V = a.V;
    const float* z = (r <= gamma) ? a.target + ((size_t)b * (gamma + 1) + r) * V
                                  : a.draft + ((size_t)b * gamma + (r - gamma - 1)) * V;
    const float it = a.inv_temp;
    float m = kNegInf, s = 0.f, best = kNegInf;
    int bi = 0x7fffffff;

    auto visit = [&](float zv, int x) {
        if (zv > best) { best = zv; bi = x; }      // visiting in increasing x per thread
        if constexpr (!GREEDY) {
            const float y = zv * it;
            if (y > m) { s = s * __expf(m - y) + 1.f; m = y; }
            else s += __expf(y - m);
        }
    };
    if ((V & 3) == 0) {
        const float4* z4 = reinterpret_cast<const float4*>(z);
        for (int j = tid; j < V / 4; j += kStatThreads) {
            const float4 v = z4[j];
            visit(v.x, 4 * j); visit(v.y, 4 * j + 1); visit(v.z, 4 * j + 2); visit(v.w, 4 * j + 3);
        }
    } else {
        for (int j = tid; j < V; j += kStatThreads) visit(z[j], j);
    }
    // wave reduce
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
        const float b2 = __shfl_xor(best, o);
        const int i2 = __shfl_xor(bi, o);
        if constexpr (!GREEDY) { const MaxSum t = ms_merge({m, s}, {m2, s2}); m = t.m; s = t.s; }
        am_merge(best, bi, b2, i2);
    }
    const int lane = tid & 63, wid = tid >> 6;
    if (lane == 0) { sm[wid] = m; ss[wid] = s; sv[wid] = best; si[wid] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kStatThreads / 64; ++w) {
            if constexpr (!GREEDY) { const MaxSum t = ms_merge({m, s}, {sm[w], ss[w]}); m = t.m; s = t.s; }
            am_merge(best, bi, sv[w], si[w]);
        }
        float zx = 0.f;
        if (!GREEDY && r != gamma) {
            const int i = (r < gamma) ? r : r - gamma - 1;
            const int x = a.tokens[(size_t)b * gamma + i];
            zx = (x >= 0 && x < V) ? z[x] * it : kNegInf;
        }
        float* st = a.stats + ((size_t)b * (2 * gamma + 1) + r) * 4;
        st[0] = GREEDY ? 0.f : m;
        st[1] = GREEDY ? 0.f : s;
        st[2] = zx;
        st[3] = (float)bi;
    }
}

struct RaceKey {
    float key;
    int x;
};

__device__ __forceinline__ void race_merge(RaceKey& a, RaceKey b) {
    if (b.key < a.key || (b.key == a.key && b.x < a.x)) a = b;
}

__global__ __launch_bounds__(kRaceThreads) void accept_decide_kernel(AcceptArgs a) {
    __shared__ int s_pos;
    __shared__ RaceKey sr[kRaceThreads / 64], sp[kRaceThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int gamma = a.gamma, V = a.V;
    const bool greedy = a.inv_temp == 0.f;
    const float* st = a.stats + (size_t)b * (2 * gamma + 1) * 4;
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    const uint32_t off = (uint32_t)a.offset;
    int32_t* out = a.out_tokens + (size_t)b * (gamma + 1);

    if (tid == 0) {
        int n = 0;
        for (; n < gamma; ++n) {
            const int x = a.tokens[(size_t)b * gamma + n];
            bool ok;
            if (greedy) {
                ok = (int)st[n * 4 + 3] == x;
            } else {
                const float* t = st + n * 4;
                const float* d = st + (gamma + 1 + n) * 4;
                const float p = __expf(t[2] - t[0]) / t[1];
                const float q = __expf(d[2] - d[0]) / d[1];
                uint32_t c0 = 0, c1 = (uint32_t)n, c2 = (uint32_t)b, c3 = off;
                philox4x32_10(c0, c1, c2, c3, k0, k1);
                ok = (x >= 0 && x < V) && philox_uniform(c0) < p / q;
            }
            if (!ok) break;
            out[n] = x;
        }
        for (int j = n + 1; j <= gamma; ++j) out[j] = -1;
        a.out_num[b] = n;
        if (greedy) out[n] = (int)st[n * 4 + 3];
        s_pos = n;
    }
    if (greedy) return;
    __syncthreads();

    const int pos = s_pos;
    const bool residual = pos < gamma;
    const float* zt = a.target + ((size_t)b * (gamma + 1) + pos) * V;
    const float* zd = residual ? a.draft + ((size_t)b * gamma + pos) * V : nullptr;
    const float* ts = st + pos * 4;
    const float* ds = residual ? st + (gamma + 1 + pos) * 4 : nullptr;
    const float it = a.inv_temp;
    RaceKey br{__builtin_huge_valf(), 0x7fffffff}, bp{__builtin_huge_valf(), 0x7fffffff};
    const int nblk = (V + 3) / 4;
    for (int j = tid; j < nblk; j += kRaceThreads) {
        uint32_t w[4] = {(uint32_t)j, (1u << 16) | (uint32_t)pos, (uint32_t)b, off};
        philox4x32_10(w[0], w[1], w[2], w[3], k0, k1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = 4 * j + e;
            if (x >= V) break;
            const float E = -__logf(philox_uniform(w[e]));
            const float pt = __expf(zt[x] * it - ts[0]) / ts[1];
            if (pt > 0.f) race_merge(bp, {E / pt, x});
            if (residual) {
                const float pd = __expf(zd[x] * it - ds[0]) / ds[1];
                const float rr = pt - pd;
                if (rr > 0.f) race_merge(br, {E / rr, x});
            }
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        race_merge(br, {__shfl_xor(br.key, o), __shfl_xor(br.x, o)});
        race_merge(bp, {__shfl_xor(bp.key, o), __shfl_xor(bp.x, o)});
    }
    const int lane = tid & 63, wid = tid >> 6;
    if (lane == 0) { sr[wid] = br; sp[wid] = bp; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kRaceThreads / 64; ++w) { race_merge(br, sr[w]); race_merge(bp, sp[w]); }
        const bool use_r = residual && br.x != 0x7fffffff;
        out[pos] = use_r ? br.x : bp.x;
    }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t s) {
    const bool greedy = a.inv_temp == 0.f;
    const int rows = greedy ? a.gamma + 1 : 2 * a.gamma + 1;
    if (greedy) accept_stats_kernel<true><<<dim3(rows, a.B), kStatThreads, 0, s>>>(a);
    else accept_stats_kernel<false><<<dim3(rows, a.B), kStatThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    accept_decide_kernel<<<a.B, kRaceThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvss
