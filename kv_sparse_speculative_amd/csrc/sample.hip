// Draft-token sampler (MagicDec Section 3.1: the draft proposes the tokens the target verifies;
// Section 5.1 drafts greedily): one token per sequence from one logit row.
//
// Sampling draws from softmax(z / t) by the exponential race argmin_x E_x / p(x), E_x = -ln u_x.
// The normaliser of p is common to every x, so the winner is argmin_x (ln E_x - z_x / t): one
// pass over the row with no statistics first. Greedy takes the argmax (ties to the lowest id).
// The statistics are kept relative to the running max of z in the base-2 domain, so that a
// block of 4 tokens costs one rescale and four exp2 with no data-dependent branch.
//   slice    grid (slice, sequence): each workgroup streams one slice of the row once with
//            16-byte loads and keeps the slice's best race key, its argmax and, when asked,
//            the slice's sum of exp(z / t - max);
//   finalize one wave per sequence merges the slices (a lane each) and writes the token and
//            statistics.
// The uniforms follow the same Philox counter layout as the acceptance race, on the draft's own
// stream: word x % 4 of block x / 4 at (stream << 16 | step, sequence, offset).

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kSampleThreads = 256;

struct SlicePart {
    float key;       // best race key of the slice
    int kx;          // its token
    float zmax;      // max z of the slice
    int imax;        // its lowest index
    float s;         // sum of 2^((z - zmax) * c), c = log2(e) / t (row statistics only)
    int pad[3];
};

__device__ __forceinline__ void key_merge(float& k, int& x, float k2, int x2) {
    if (k2 < k || (k2 == k && x2 < x)) { k = k2; x = x2; }
}
__device__ __forceinline__ void max_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
// (max, sum) pairs in the base-2 domain: s = sum 2^((z - zmax) * c).
__device__ __forceinline__ float sum_merge(float z1, float s1, float z2, float s2, float c) {
    const float M = fmaxf(z1, z2);
    if (M == kNegInf) return 0.f;
    return s1 * __builtin_amdgcn_exp2f((z1 - M) * c) + s2 * __builtin_amdgcn_exp2f((z2 - M) * c);
}

// Per-thread state of one slice. Each thread visits its tokens in increasing order, so a later
// token replaces the best only when strictly better and ties keep the lowest id. Only entries
// above -inf are tracked; a row without one is rescanned by the finalize kernel.
template <bool SAMPLE, bool STATS>
struct SliceState {
    float bk = __builtin_huge_valf(), best = kNegInf, s = 0.f;
    int bx = 0x7fffffff, bi = 0x7fffffff;

    // One block of 4 tokens x = 4j .. 4j + 3; `n` of them are in the row (4 but at the end).
    // Race key of token x: log2(-log2 u_x) - z_x * c, which orders tokens as ln E_x - z_x / t
    // does (E_x = -ln u_x): both are log2(e) times the latter plus the constant log2(ln 2).
    template <bool CHECK>
    __device__ __forceinline__ void visit(const float (&v)[4], int j, int n, uint32_t w1,
                                          uint32_t w2, uint32_t w3, uint32_t k0, uint32_t k1,
                                          float c) {
        float bmax = best;
        if constexpr (STATS) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!CHECK || e < n) bmax = fmaxf(bmax, v[e]);
            // rescale the running sum to the new maximum, then add the block's terms
            if (bmax != kNegInf) {
                float t = s * __builtin_amdgcn_exp2f((best - bmax) * c);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!CHECK || e < n) t += __builtin_amdgcn_exp2f((v[e] - bmax) * c);
                s = t;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if ((!CHECK || e < n) && v[e] > best) { best = v[e]; bi = 4 * j + e; }
        if constexpr (SAMPLE) {
            uint32_t w[4] = {(uint32_t)j, w1, w2, w3};
            philox4x32_10(w[0], w[1], w[2], w[3], k0, k1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lu = __builtin_amdgcn_logf(philox_uniform(w[e]));     // log2 u < 0
                const float key = fmaf(-v[e], c, __builtin_amdgcn_logf(-lu));
                if ((!CHECK || e < n) && key < bk) { bk = key; bx = 4 * j + e; }
            }
        }
    }
};

template <bool SAMPLE, bool STATS>
__global__ __launch_bounds__(kSampleThreads) void sample_slice_kernel(SampleArgs a, SlicePart* parts,
                                                                      int nslice) {
    __shared__ SlicePart sp[kSampleThreads / 64];
    const int slice = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const float* z = a.logits + (size_t)b * a.V;
    const int nblk = (a.V + 3) / 4;                          // blocks of 4 tokens
    const int per = (nblk + nslice - 1) / nslice;
    const int j0 = slice * per, j1 = min(nblk, j0 + per);
    const float c = a.inv_temp * kLog2e;
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    const uint32_t w1 = ((uint32_t)a.stream_id << 16) | (uint32_t)a.step;
    const uint32_t w2 = (uint32_t)b, w3 = (uint32_t)a.offset;
    SliceState<SAMPLE, STATS> st;
    constexpr int kBatch = 4;                                // 16-byte loads in flight per thread
    int j = j0 + tid;
    // whole blocks of 4 read as one 16-byte load when the row allows it, kBatch at a time
    if ((a.V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0) {
        const float4* z4 = reinterpret_cast<const float4*>(z);
        for (; j + (kBatch - 1) * kSampleThreads < j1; j += kBatch * kSampleThreads) {
            float v[kBatch][4];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const float4 f = load_stream_f4(z4 + j + q * kSampleThreads);
                v[q][0] = f.x; v[q][1] = f.y; v[q][2] = f.z; v[q][3] = f.w;
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                st.template visit<false>(v[q], j + q * kSampleThreads, 4, w1, w2, w3, k0, k1, c);
        }
        for (; j < j1; j += kSampleThreads) {
            const float4 f = load_stream_f4(z4 + j);
            const float v[4] = {f.x, f.y, f.z, f.w};
            st.template visit<false>(v, j, 4, w1, w2, w3, k0, k1, c);
        }
    } else {
        for (; j < j1; j += kSampleThreads) {
            const int n = min(4, a.V - 4 * j);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = z[min(4 * j + e, a.V - 1)];
            st.template visit<true>(v, j, n, w1, w2, w3, k0, k1, c);
        }
    }
    float bk = st.bk, best = st.best, s = st.s;
    int bx = st.bx, bi = st.bi;
    for (int o = 32; o > 0; o >>= 1) {
        const float best2 = __shfl_xor(best, o);
        if constexpr (STATS) s = sum_merge(best, s, best2, __shfl_xor(s, o), c);
        if constexpr (SAMPLE) key_merge(bk, bx, __shfl_xor(bk, o), __shfl_xor(bx, o));
        max_merge(best, bi, best2, __shfl_xor(bi, o));
    }
    const int lane = tid & 63, wid = tid >> 6;
    if (lane == 0) sp[wid] = SlicePart{bk, bx, best, bi, s, {0, 0, 0}};
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kSampleThreads / 64; ++w) {
            if constexpr (STATS) s = sum_merge(best, s, sp[w].zmax, sp[w].s, c);
            if constexpr (SAMPLE) key_merge(bk, bx, sp[w].key, sp[w].kx);
            max_merge(best, bi, sp[w].zmax, sp[w].imax);
        }
        parts[(size_t)b * nslice + slice] = SlicePart{bk, bx, best, bi, s, {0, 0, 0}};
    }
}

__global__ __launch_bounds__(64) void sample_finalize_kernel(SampleArgs a, const SlicePart* parts,
                                                             int nslice) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const float c = a.inv_temp * kLog2e;
    float bk = __builtin_huge_valf(), best = kNegInf, s = 0.f;
    int bx = 0x7fffffff, bi = 0x7fffffff;
    for (int k = lane; k < nslice; k += 64) {
        const SlicePart p = parts[(size_t)b * nslice + k];
        s = sum_merge(best, s, p.zmax, p.s, c);
        key_merge(bk, bx, p.key, p.kx);
        max_merge(best, bi, p.zmax, p.imax);
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float best2 = __shfl_xor(best, o);
        s = sum_merge(best, s, best2, __shfl_xor(s, o), c);
        key_merge(bk, bx, __shfl_xor(bk, o), __shfl_xor(bx, o));
        max_merge(best, bi, best2, __shfl_xor(bi, o));
    }
    // The argmax is over the non-NaN entries: a row in which no entry exceeds -inf has its
    // argmax at its first non-NaN entry (-1 if none), found by a scan of the whole wave.
    int arg = bi;
    if (bi == 0x7fffffff) {
        const float* z = a.logits + (size_t)b * a.V;
        arg = -1;
        for (int x0 = 0; x0 < a.V; x0 += 64) {          // wave-uniform trip count
            const int x = x0 + lane;
            const float v = x < a.V ? z[x] : __builtin_nanf("");
            int f = v == v ? x : 0x7fffffff;
            for (int o = 32; o > 0; o >>= 1) f = min(f, __shfl_xor(f, o));
            if (f != 0x7fffffff) { arg = f; break; }
        }
    }
    if (lane != 0) return;
    const bool sample = a.inv_temp != 0.f;
    a.tokens[b] = sample ? bx : arg;
    if (a.stats != nullptr) {
        // max of z / t is (max z) / t: rounding is monotone, so the two agree exactly
        float* o = a.stats + (size_t)b * 4;
        o[0] = sample ? best * a.inv_temp : 0.f;
        o[1] = sample ? s : 0.f;
        o[2] = 0.f;
        o[3] = (float)arg;
    }
}

}  // namespace

int sample_slices(int V) { return V >= 8192 ? (V + 8191) / 8192 : 1; }

size_t sample_workspace_bytes(int B, int V) {
    return (size_t)B * sample_slices(V) * sizeof(SlicePart);
}

hipError_t launch_sample(const SampleArgs& a, void* ws, hipStream_t s) {
    const int nslice = sample_slices(a.V);
    SlicePart* parts = static_cast<SlicePart*>(ws);
    const dim3 grid(nslice, a.B);
    const bool sample = a.inv_temp != 0.f, stats = sample && a.stats != nullptr;
    if (!sample) sample_slice_kernel<false, false><<<grid, kSampleThreads, 0, s>>>(a, parts, nslice);
    else if (stats) sample_slice_kernel<true, true><<<grid, kSampleThreads, 0, s>>>(a, parts, nslice);
    else sample_slice_kernel<true, false><<<grid, kSampleThreads, 0, s>>>(a, parts, nslice);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    sample_finalize_kernel<<<a.B, 64, 0, s>>>(a, parts, nslice);
    return hipGetLastError();
}

}  // namespace kvss
