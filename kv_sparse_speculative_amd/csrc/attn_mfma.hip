// bf16 split-KV attention on gfx950 matrix cores: verify (gamma + 1 causal queries per
// sequence over the full cache) and sparse draft (one query over a gathered subset).
//
// MagicDec (arXiv 2408.11049v5) Section 3.2 explains why this is the hot path: in the
// long-context, large-batch regime the per-step KV load dominates, and verification costs
// about one decode because both stream the same cache. The kernel therefore streams each
// (sequence, KV head)'s K and V exactly once per launch and keeps all G * T query rows of
// that KV head (GQA, Section 3.2) on the same bytes.
//
// Work decomposition: grid (split, KV head, sequence); 4 waves per workgroup; each wave takes
// 32-key chunks of the split round-robin. Per chunk and wave:
//   S^T (16 keys x 16 rows tiles) = K . Q^T   with v_mfma_f32_16x16x32_bf16: K rows come
//       straight from HBM as the A operand (16 B per lane, one key row per 16 lanes), Q^T is
//       resident in registers as the B operand;
//   online softmax in the log2 domain (row max/sum across the 4 lane groups with xor
//       shuffles; each lane owns one query row of the C tile);
//   O^T (16 dims x 16 rows) += V^T . P^T  with P split into bf16 hi + lo parts (two MFMAs) so
//       that P carries ~16 mantissa bits; V^T is read transposed from a padded LDS tile
//       that the same wave wrote.
// Waves merge (max, sum, O) through LDS; with one split the workgroup writes the final
// normalised output, otherwise (m, l, o) partials that the merge kernel combines.

#include "common.h"
#include "launch.h"

namespace kvss {
namespace {

constexpr int kWaves = 4;

template <int D>
struct MfmaCfg {
    static constexpr int KS = D / 32;          // k-steps of the QK^T contraction
    static constexpr int DT = D / 16;          // dim tiles of the PV product
    static constexpr int STRIDE = D + 4;       // LDS row stride in bf16 (row = D/2 + 2 dwords)
    static constexpr int VLDS = kWaves * 32 * STRIDE * 2;            // bytes
    static constexpr int MERGE = kWaves * 32 * (D + 2) * 4;          // bytes
    static constexpr int SMEM = VLDS > MERGE ? VLDS : MERGE;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
    bf16x8 r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

template <int D, bool GATHER>
__global__ __launch_bounds__(kWaves * 64) void attn_mfma_kernel(AttnArgs a) {
    using C = MfmaCfg<D>;
    constexpr int KS = C::KS, DT = C::DT, STRIDE = C::STRIDE;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
    __shared__ int s_bad;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (threadIdx.x == 0) s_bad = 0;

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
    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);

    // Q^T as the B operand: lane supplies column (row) rt*16 + m16, dims ks*32 + q4*8 .. +7.
    bf16x8 qop[2][KS];
    int limit[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = rt * 16 + m16;
        limit[rt] = -1;
        if (r < a.R) {
            const int h = g * a.G + r / a.T, t = r % a.T;
            const uint16_t* src = qp + (((size_t)b * a.Hq + h) * a.T + t) * D + q4 * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qop[rt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(src + ks * 32));
            limit[rt] = GATHER ? 0x7fffffff : L - a.T + t;
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qop[rt][ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }

    f32x4 o[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][0] = o[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow[2] = {kNegInf, kNegInf};
    float lrow[2] = {0.f, 0.f};
    bool bad = false;

    uint16_t* vl = reinterpret_cast<uint16_t*>(smem) + wid * 32 * STRIDE;
    const int32_t* sel = GATHER ? a.sel_idx + ((size_t)b * a.Hkv + g) * a.k_max : nullptr;

    for (int c0 = v_begin + wid * 32; c0 < v_end; c0 += kWaves * 32) {
        uint4 kr[2][KS], vr[2][KS];
        unsigned okmask[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int v = c0 + kt * 16 + m16;
            bool ok = v < v_end;
            int pos = v;
            if constexpr (GATHER) {
                if (ok) {
                    if (v < n_list) {
                        pos = sel[v];
                        ok = (pos >= 0) && (pos < lo);
                    } else {
                        pos = lo + (v - n_list);
                    }
                }
            }
            size_t off = 0;
            if (ok) {
                if (!cache.row_offset(b, g, pos, off)) { bad = true; ok = false; }
            }
            okmask[kt] = (unsigned)(__ballot(ok) & 0xffffull);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ok) {
                    kr[kt][ks] = *reinterpret_cast<const uint4*>(kp + off + ks * 32 + q4 * 8);
                    vr[kt][ks] = *reinterpret_cast<const uint4*>(vp + off + ks * 32 + q4 * 8);
                } else {
                    kr[kt][ks] = make_uint4(0, 0, 0, 0);
                    vr[kt][ks] = make_uint4(0, 0, 0, 0);
                }
            }
        }

        // V rows -> this wave's LDS tile (row = key within chunk).
        wave_lds_order();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *reinterpret_cast<uint4*>(vl + (kt * 16 + m16) * STRIDE + ks * 32 + q4 * 8) = vr[kt][ks];

        // S^T = K . Q^T : C tile [key 4*q4+i][row m16].
        f32x4 sacc[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[kt][ks]), qop[rt][ks],
                                                                 acc, 0, 0, 0);
                sacc[kt][rt] = acc;
            }

        bf16x8 phi[2], plo[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float sv[8];
            float cmax = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = kt * 16 + q4 * 4 + i;
                    bool allowed = (okmask[kt] >> (q4 * 4 + i)) & 1u;
                    if constexpr (!GATHER) allowed = allowed && (c0 + key <= limit[rt]);
                    const float x = allowed ? sacc[kt][rt][i] * a.scale_log2 : kNegInf;
                    sv[kt * 4 + i] = x;
                    cmax = fmaxf(cmax, x);
                }
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
            const float mnew = fmaxf(mrow[rt], cmax);
            const float muse = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrow[rt] - muse);
            mrow[rt] = mnew;
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(sv[j] - muse);
                const __bf16 hi = (__bf16)p;
                phi[rt][j] = hi;
                plo[rt][j] = (__bf16)(p - (float)hi);
                psum += p;
            }
            lrow[rt] = lrow[rt] * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
        }

        // O^T += V^T . P^T. k-slot j of lane group q4 is key 16*(j/4) + 4*q4 + (j%4), matching
        // the C-tile keys this lane holds in sacc[j/4][*][j%4].
        wave_lds_order();
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int k0 = 16 * (p >> 1) + 4 * q4 + 2 * (p & 1);    // slot j = 2p
                w[p] = (uint32_t)vl[k0 * STRIDE + dt * 16 + m16] |
                       ((uint32_t)vl[(k0 + 1) * STRIDE + dt * 16 + m16] << 16);
            }
            const bf16x8 av = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi[rt], o[dt][rt], 0, 0, 0);
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo[rt], o[dt][rt], 0, 0, 0);
            }
        }
        wave_lds_order();
    }

    // Row sums were kept per lane group; complete them.
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        lrow[rt] += __shfl_xor(lrow[rt], 16);
        lrow[rt] += __shfl_xor(lrow[rt], 32);
    }

    __syncthreads();                 // every wave is done with its V tile (smem is reused)
    if (__ballot(bad) != 0ull && lane == 0) s_bad = 1;
    float* so = reinterpret_cast<float*>(smem);               // [wave][32 rows][D]
    float* sml = so + kWaves * 32 * D;                         // [wave][32 rows][2]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(wid * 32 + rt * 16 + m16) * D + dt * 16 + q4 * 4 + i] = o[dt][rt][i];
    if (q4 == 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            sml[(wid * 32 + rt * 16 + m16) * 2 + 0] = mrow[rt];
            sml[(wid * 32 + rt * 16 + m16) * 2 + 1] = lrow[rt];
        }
    }
    __syncthreads();

    const bool poisoned = s_bad != 0;
    const float qnan = __builtin_nanf("");
    for (int idx = threadIdx.x; idx < a.R * D; idx += kWaves * 64) {
        const int r = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sml[(w * 32 + r) * 2]);
        float lsum = 0.f, osum = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float e = __builtin_amdgcn_exp2f(sml[(w * 32 + r) * 2] - M);
                lsum += e * sml[(w * 32 + r) * 2 + 1];
                osum += e * so[(w * 32 + r) * D + d];
            }
        }
        const int h = g * a.G + r / a.T, t = r % a.T;
        const size_t row = ((size_t)b * a.Hq + h) * a.T + t;
        if (a.nsplit == 1) {
            float ov = lsum > 0.f ? osum / lsum : 0.f;
            if (poisoned) ov = qnan;
            a.out[row * D + d] = ov;
            if (d == 0 && a.lse != nullptr) {
                float lv = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : kNegInf;
                a.lse[row] = poisoned ? qnan : lv;
            }
        } else {
            float* pp = a.part + (row * a.nsplit + split) * (D + 2);
            pp[d] = poisoned ? qnan : osum;
            if (d == 0) {
                pp[D] = poisoned ? qnan : M;
                pp[D + 1] = poisoned ? qnan : lsum;
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, bool gather, hipStream_t s) {
    dim3 grid(a.nsplit, a.Hkv, a.B), block(kWaves * 64);
    if (a.D == 128) {
        if (gather) attn_mfma_kernel<128, true><<<grid, block, 0, s>>>(a);
        else attn_mfma_kernel<128, false><<<grid, block, 0, s>>>(a);
    } else {
        if (gather) attn_mfma_kernel<64, true><<<grid, block, 0, s>>>(a);
        else attn_mfma_kernel<64, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace kvss
