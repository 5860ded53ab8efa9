// float32 split-KV attention on the vector ALU (verify and sparse draft over fp32 caches).
//
// Same contract and split/partial format as the bf16 matrix-core kernel (MagicDec
// Sections 3.1-3.2: verify of gamma + 1 causal queries; Section 4.1 Eq. (3): draft over a
// sparse set), for caches stored in float32. One wave per (split, KV head, sequence); lane r
// owns query row r (R <= 32 <= 64 lanes) and keeps its running max, sum and output in
// registers; 32-key tiles of K and V are staged through LDS and read as broadcasts.

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

template <int D, bool GATHER>
__global__ __launch_bounds__(64) void attn_simple_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) float ks[32][D];
    __shared__ __attribute__((aligned(16))) float vs[32][D];
    __shared__ int spos[32];
    __shared__ long long soff[32];

    const int lane = threadIdx.x;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = max(min(a.kv_lens[b], a.max_kv_len), 0);
    int n_list = 0, lo = 0;
    if constexpr (GATHER) {
        n_list = min(max(a.sel_count[b], 0), a.k_max);
        lo = min(max(a.tail_lo[b], 0), L);
    }
    const int total = n_list + (L - lo);
    const int v_begin = split * a.split_len;
    const int v_end = (split == a.nsplit - 1) ? total : min(v_begin + a.split_len, total);
    const PagedCache cache{a.block_table, a.Hkv, a.bs, a.max_blocks, a.num_blocks, D};
    const float* kp = static_cast<const float*>(a.k);
    const float* vp = static_cast<const float*>(a.v);
    const float* qp = static_cast<const float*>(a.q);
    const int32_t* sel = GATHER ? a.sel_idx + ((size_t)b * a.Hkv + g) * a.k_max : nullptr;

    const bool row_ok = lane < a.R;
    const int h = g * a.G + (row_ok ? lane / a.T : 0), t = row_ok ? lane % a.T : 0;
    const size_t row = ((size_t)b * a.Hq + h) * a.T + t;
    const int limit = GATHER ? 0x7fffffff : L - a.T + t;
    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = row_ok ? qp[row * D + d] : 0.f;
        o[d] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    bool bad = false;

    for (int c0 = v_begin; c0 < v_end; c0 += 32) {
        if (lane < 32) {
            const int v = c0 + lane;
            bool ok = v < v_end;
            int pos = v;
            if constexpr (GATHER) {
                if (ok) {
                    if (v < n_list) { pos = sel[v]; ok = pos >= 0 && pos < lo; }
                    else pos = lo + (v - n_list);
                }
            }
            size_t off = 0;
            if (ok && !cache.row_offset(b, g, pos, off)) { bad = true; ok = false; }
            spos[lane] = ok ? pos : -1;
            soff[lane] = (long long)off;
        }
        __syncthreads();
        for (int idx = lane; idx < 32 * (D / 4); idx += 64) {
            const int j = idx / (D / 4), c = idx % (D / 4);
            float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
            if (spos[j] >= 0) {
                kv4 = *reinterpret_cast<const float4*>(kp + soff[j] + c * 4);
                vv4 = *reinterpret_cast<const float4*>(vp + soff[j] + c * 4);
            }
            *reinterpret_cast<float4*>(&ks[j][c * 4]) = kv4;
            *reinterpret_cast<float4*>(&vs[j][c * 4]) = vv4;
        }
        __syncthreads();
        if (row_ok) {
            for (int j = 0; j < 32; ++j) {
                const int pos = spos[j];
                if (pos < 0 || pos > limit) continue;
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[j][d], s);
                s *= a.scale_log2;
                const float mnew = fmaxf(m, s);
                const float alpha = __builtin_amdgcn_exp2f(m - mnew);
                const float p = __builtin_amdgcn_exp2f(s - mnew);
                l = l * alpha + p;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[j][d], o[d] * alpha);
                m = mnew;
            }
        }
        __syncthreads();
    }

    const bool poisoned = __ballot(bad) != 0ull;
    if (!row_ok) return;
    const float qnan = __builtin_nanf("");
    if (a.nsplit == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) a.out[row * D + d] = poisoned ? qnan : o[d] * inv;
        if (a.lse) a.lse[row] = poisoned ? qnan : (l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf);
    } else {
        float* pp = a.part + (row * a.nsplit + split) * (D + 2);
#pragma unroll
        for (int d = 0; d < D; ++d) pp[d] = poisoned ? qnan : o[d];
        pp[D] = poisoned ? qnan : m;
        pp[D + 1] = poisoned ? qnan : l;
    }
}

}  // namespace

hipError_t launch_attn_simple(const AttnArgs& a, bool gather, hipStream_t s) {
    dim3 grid(a.nsplit, a.Hkv, a.B), block(64);
    if (a.D == 128) {
        if (gather) attn_simple_kernel<128, true><<<grid, block, 0, s>>>(a);
        else attn_simple_kernel<128, false><<<grid, block, 0, s>>>(a);
    } else {
        if (gather) attn_simple_kernel<64, true><<<grid, block, 0, s>>>(a);
        else attn_simple_kernel<64, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace kvss
