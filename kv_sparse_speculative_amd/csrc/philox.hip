// The library's counter-based generator evaluated on caller-given counters: the same device
// Philox4x32-10 that the acceptance race and the draft sampler draw from, so a caller can
// replay a draw (the counter layout is documented with spec_accept and draft_sample).

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kPhiloxThreads = 256;

__global__ __launch_bounds__(kPhiloxThreads) void philox_kernel(const uint4* __restrict__ ctr,
                                                                int64_t n, uint32_t k0,
                                                                uint32_t k1, uint4* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kPhiloxThreads + threadIdx.x;
    if (i >= n) return;
    uint4 c = ctr[i];
    philox4x32_10(c.x, c.y, c.z, c.w, k0, k1);
    out[i] = c;
}

}  // namespace

hipError_t launch_philox(const uint32_t* counters, int64_t n, uint64_t seed, uint32_t* out,
                         hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + kPhiloxThreads - 1) / kPhiloxThreads;
    philox_kernel<<<(unsigned)blocks, kPhiloxThreads, 0, s>>>(
        reinterpret_cast<const uint4*>(counters), n, (uint32_t)seed, (uint32_t)(seed >> 32),
        reinterpret_cast<uint4*>(out));
    return hipGetLastError();
}

}  // namespace kvss
