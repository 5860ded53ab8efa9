// Device-side helpers shared by the kvss kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Widen the 8 bf16 values packed in a 16-byte vector to float.
__device__ __forceinline__ void widen8(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// 16-byte load of data the call reads exactly once (K/V rows, logits): a nontemporal load.
// On gfx950 a stream of these keeps ~7.1 TB/s of HBM read rate, against ~6.2 TB/s for plain
// loads that allocate in the caches.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
    const u32x4_t t = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 load_stream_f4(const void* p) {
    const uint4 u = load_stream(p);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
}

// Compiler-level memory barrier: keeps LDS stores and the loads that read them (from other
// lanes of the same wave) in program order; the LDS unit executes one wave's DS instructions
// in order, so no hardware wait is needed between them.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// x / bs with a shift when the block size is a power of two (sh >= 0), else a division.
__device__ __forceinline__ int div_bs(int x, int bs, int sh) { return sh >= 0 ? x >> sh : x / bs; }

// Physical row address of logical position `pos` of (sequence, KV head) in the paged cache.
// Returns false when the block id read from the table is outside [0, num_blocks).
struct PagedCache {
    const int32_t* table;   // [B, max_blocks]
    int Hkv, bs, max_blocks, num_blocks, D;

    __device__ __forceinline__ bool row_offset(int b, int g, int pos, size_t& off) const {
        const int blk = table[(size_t)b * max_blocks + pos / bs];
        off = (((size_t)blk * Hkv + g) * bs + (pos % bs)) * (size_t)D;
        return (unsigned)blk < (unsigned)num_blocks;
    }
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11): ten rounds of two 32x32->64 multiplies with the paper's multipliers, the key bumped
// by its Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              uint32_t k0, uint32_t k1) {
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        // one 32x32->64 multiply-add instruction per product gives both halves
        const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
    }
}

// 32-bit word -> uniform in (0, 1): (x >> 9) * 2^-23 + 2^-24, exact in binary32.
__device__ __forceinline__ float philox_uniform(uint32_t x) {
    return (float)(x >> 9) * 0x1p-23f + 0x1p-24f;
}

}  // namespace kvss
