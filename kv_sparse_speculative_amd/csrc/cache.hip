// KV-cache maintenance: appending new rows to a paged cache and materialising the compressed
// draft cache (MagicDec Section 3.1: the gamma + 1 verified tokens join the cache the verify
// pass reads; Appendix A.1, Fig. 8: the static compressed KV is built at prefill and the draft
// decodes over it).
//
// Both are plain row copies: every K or V row is moved as 16-byte vector loads and stores by
// consecutive lanes (a bf16 row of 128 dims is 16 lanes), so each wave moves four whole rows
// per instruction and the copies run at the HBM copy rate.

#include "common.h"
#include "kvss.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kCopyThreads = 256;
constexpr unsigned kNoRow = 0xffffffffu;

// ---------------------------------------------------------------- append
// One workgroup per (sequence, new row t): the Hkv K rows and Hkv V rows of that token.
__global__ __launch_bounds__(kCopyThreads) void kv_append_kernel(AppendArgs a) {
    const int b = blockIdx.x / a.T, t = blockIdx.x % a.T;
    const long pos = (long)a.start[b] + t;
    if (pos < 0 || pos >= (long)a.max_blocks * a.bs) return;
    const int blk = a.block_table[(size_t)b * a.max_blocks + pos / a.bs];
    if ((unsigned)blk >= (unsigned)a.num_blocks) return;
    const int row16 = a.row_bytes / 16;                       // 16-byte pieces per row
    const int per = a.Hkv * row16;                            // pieces of K (and of V)
    const uint4* kn = static_cast<const uint4*>(a.k_new);
    const uint4* vn = static_cast<const uint4*>(a.v_new);
    uint4* kc = static_cast<uint4*>(a.k);
    uint4* vc = static_cast<uint4*>(a.v);
    for (int i = threadIdx.x; i < 2 * per; i += kCopyThreads) {
        const int which = i >= per, j = which ? i - per : i;
        const int g = j / row16, c = j % row16;
        const size_t src = (((size_t)b * a.Hkv + g) * a.T + t) * row16 + c;
        const size_t dst = (((size_t)blk * a.Hkv + g) * a.bs + pos % a.bs) * row16 + c;
        if (which) vc[dst] = load_stream(vn + src);
        else kc[dst] = load_stream(kn + src);
    }
}

// ---------------------------------------------------------------- compact draft cache
// Grid (row chunk, KV head, sequence); each workgroup copies kCompactRows slots of (b, g).
constexpr int kCompactRows = 64;

__global__ __launch_bounds__(kCopyThreads) void compact_build_kernel(CompactArgs a) {
    __shared__ unsigned s_src[kCompactRows], s_dst[kCompactRows];
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = max(min(a.kv_lens[b], a.max_kv_len), 0);
    const int lo = min(max(a.tail_lo[b], 0), L);
    const int n = a.k_max > 0 ? min(max(a.sel_count[b], 0), a.k_max) : 0;
    int tail = L - lo;
    const bool poison = tail > a.max_tail;           // the caller's bound on the tail is broken
    if (poison) tail = a.max_tail;
    const int total = n + tail;
    if (chunk == 0 && g == 0 && threadIdx.x == 0) a.dst_lens[b] = total;
    const int j0 = chunk * kCompactRows;
    if (j0 >= total) return;
    const int rows = min(kCompactRows, total - j0);

    // Slot -> source row (kNoRow: write NaN) and destination row (kNoRow: not written).
    if (threadIdx.x < rows) {
        const int j = j0 + threadIdx.x;
        unsigned src = kNoRow, dst = kNoRow;
        const int p = j < n ? a.sel_idx[((size_t)b * a.Hkv + g) * a.k_max + j] : lo + (j - n);
        if (!poison && (j >= n || (p >= 0 && p < lo))) {
            const int blk = a.block_table[(size_t)b * a.max_blocks + p / a.bs];
            if ((unsigned)blk < (unsigned)a.num_blocks)
                src = ((unsigned)blk * a.Hkv + g) * a.bs + (unsigned)(p % a.bs);
        }
        const int dblk = a.dst_table[(size_t)b * a.dst_max_blocks + j / a.dst_bs];
        if ((unsigned)dblk < (unsigned)a.dst_num_blocks)
            dst = ((unsigned)dblk * a.Hkv + g) * a.dst_bs + (unsigned)(j % a.dst_bs);
        s_src[threadIdx.x] = src;
        s_dst[threadIdx.x] = dst;
    }
    __syncthreads();

    const int row16 = a.row_bytes / 16;
    const uint4 nan4 = a.dtype == KVSS_BF16 ? make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u)
                                            : make_uint4(0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u);
    const uint4* ks = static_cast<const uint4*>(a.k);
    const uint4* vs = static_cast<const uint4*>(a.v);
    uint4* kd = static_cast<uint4*>(a.dst_k);
    uint4* vd = static_cast<uint4*>(a.dst_v);
    for (int i = threadIdx.x; i < rows * row16; i += kCopyThreads) {
        const int r = i / row16, c = i % row16;
        const unsigned src = s_src[r], dst = s_dst[r];
        if (dst == kNoRow) continue;
        uint4 kv = nan4, vv = nan4;
        if (src != kNoRow) {
            kv = load_stream(ks + (size_t)src * row16 + c);
            vv = load_stream(vs + (size_t)src * row16 + c);
        }
        kd[(size_t)dst * row16 + c] = kv;
        vd[(size_t)dst * row16 + c] = vv;
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
    kv_append_kernel<<<a.B * a.T, kCopyThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_compact_build(const CompactArgs& a, hipStream_t s) {
    // At least one chunk, so the lengths are written even when there is nothing to copy.
    const int chunks = max((a.k_max + a.max_tail + kCompactRows - 1) / kCompactRows, 1);
    compact_build_kernel<<<dim3(chunks, a.Hkv, a.B), kCopyThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvss
