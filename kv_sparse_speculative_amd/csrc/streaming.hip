// StreamingLLM draft set (MagicDec Section 5.1: StreamingLLM-style sparse KV for drafting;
// Table 1: budget 512) in the sparse-draft encoding: the `sink` first rows as the selected
// list and the most recent `window` rows as the dense tail [max(sink, L - window), L).

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

__global__ __launch_bounds__(256) void streaming_set_kernel(const int32_t* kv_lens, int Hkv,
                                                            int sink, int window,
                                                            int32_t* sel_idx, int32_t* sel_count,
                                                            int32_t* tail_lo) {
    const int b = blockIdx.x;
    const int L = max(kv_lens[b], 0);
    const int n = min(sink, L);
    for (int idx = threadIdx.x; idx < Hkv * sink; idx += blockDim.x) {
        const int j = idx % sink;
        sel_idx[(size_t)b * Hkv * sink + idx] = j < n ? j : -1;
    }
    if (threadIdx.x == 0) {
        sel_count[b] = n;
        tail_lo[b] = max(sink, L - window);
    }
}

// tail_lo[b] = max(min(kv_lens[b], max_kv_len) - back, 0): the start of the last `back` rows.
__global__ __launch_bounds__(256) void tail_lo_kernel(const int32_t* kv_lens, int B, int max_kv_len,
                                                      int back, int32_t* tail_lo) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b < B) tail_lo[b] = max(min(kv_lens[b], max_kv_len) - back, 0);
}

}  // namespace

hipError_t launch_tail_lo(const int32_t* kv_lens, int B, int max_kv_len, int back, int32_t* tail_lo,
                          hipStream_t s) {
    if (B == 0) return hipSuccess;
    tail_lo_kernel<<<(B + 255) / 256, 256, 0, s>>>(kv_lens, B, max_kv_len, back, tail_lo);
    return hipGetLastError();
}

hipError_t launch_streaming_set(const int32_t* kv_lens, int B, int Hkv, int sink, int window,
                                int32_t* sel_idx, int32_t* sel_count, int32_t* tail_lo,
                                hipStream_t s) {
    if (B == 0) return hipSuccess;
    streaming_set_kernel<<<B, 256, 0, s>>>(kv_lens, Hkv, sink, window, sel_idx, sel_count, tail_lo);
    return hipGetLastError();
}

}  // namespace kvss
