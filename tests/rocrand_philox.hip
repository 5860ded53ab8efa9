// Test helper (not part of the library): rocRAND's device Philox4x32-10 on caller counters,
// a third implementation next to the library's and the oracle's. Counter (c0, c1, c2, c3) is
// reached through rocRAND's documented state layout: subsequence c2 + 2^32 c3 (a subsequence
// spans 4 * 2^64 numbers) and absolute offset 4 * (c0 + 2^32 c1) numbers into it.

#include <hip/hip_runtime.h>
#include <rocrand/rocrand_kernel.h>
#include <stdint.h>

__global__ void rocrand_philox_kernel(const uint4* ctr, int64_t n, unsigned long long seed,
                                      uint4* out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint4 c = ctr[i];
    rocrand_state_philox4x32_10 st;
    const unsigned long long subsequence = (unsigned long long)c.z | ((unsigned long long)c.w << 32);
    const unsigned long long offset = 4ull * ((unsigned long long)c.x | ((unsigned long long)c.y << 32));
    rocrand_init(seed, subsequence, offset, &st);
    out[i] = rocrand4(&st);
}

extern "C" int rocrand_philox(const void* counters, int64_t n, unsigned long long seed, void* out) {
    if (n <= 0) return 0;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    rocrand_philox_kernel<<<blocks, 256>>>(static_cast<const uint4*>(counters), n, seed,
                                           static_cast<uint4*>(out));
    if (hipGetLastError() != hipSuccess) return -1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
