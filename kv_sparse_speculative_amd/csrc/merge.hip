// Split-KV merge: combine per-split softmax partials (max m_s, sum l_s, unnormalised o_s,
// all in the log2 domain) into the normalised output and the natural-log LSE.
// M = max_s m_s, Lambda = sum_s 2^(m_s - M) l_s, O = sum_s 2^(m_s - M) o_s / Lambda,
// LSE = (M + log2 Lambda) * ln 2. Flash-decoding-style partitioning is cited by MagicDec
// (Section 2) as the system optimisation for decode latency; this is its combine step.

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part, int nsplit,
                                                    int D, float* __restrict__ out,
                                                    float* __restrict__ lse) {
    const size_t row = blockIdx.x;
    const float* p = part + row * nsplit * (size_t)(D + 2);
    float M = kNegInf;
    bool nan = false;
    for (int s = 0; s < nsplit; ++s) {
        const float ms = p[s * (D + 2) + D];
        nan |= ms != ms;
        M = fmaxf(M, ms);
    }
    const float qnan = __builtin_nanf("");
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float lam = 0.f, o = 0.f;
        if (M != kNegInf) {
            for (int s = 0; s < nsplit; ++s) {
                const float* ps = p + s * (D + 2);
                if (ps[D] == kNegInf) continue;
                const float e = __builtin_amdgcn_exp2f(ps[D] - M);
                lam += e * ps[D + 1];
                o += e * ps[d];
            }
        }
        out[row * D + d] = nan ? qnan : (lam > 0.f ? o / lam : 0.f);
        if (d == 0 && lse != nullptr)
            lse[row] = nan ? qnan : (lam > 0.f ? (M + __log2f(lam)) * kLn2 : kNegInf);
    }
}

}  // namespace

hipError_t launch_merge(const float* part, int rows, int nsplit, int D, float* out, float* lse,
                        hipStream_t s) {
    if (rows == 0) return hipSuccess;
    merge_kernel<<<rows, 128, 0, s>>>(part, nsplit, D, out, lse);
    return hipGetLastError();
}

}  // namespace kvss
