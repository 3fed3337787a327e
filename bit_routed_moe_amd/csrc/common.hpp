// Shared device helpers for the ds4moe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4 {

constexpr int WAVE = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
    return __uint_as_float(bits << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> packed bf16 pair (lo = a, hi = b), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// IEEE binary16 bit pattern -> fp32 (exact, subnormals included).
__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float silu_f32(float g) {
    return g / (1.0f + __expf(-g));
}

// Butterfly sum over the whole wave (fixed order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Butterfly sum inside aligned groups of `width` lanes (width a power of 2 <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}

// Order-preserving 64-bit key: high word = float bits mapped so that unsigned
// order equals numeric order (-0 folded into +0), low word = ~index so that
// equal values rank the lower index higher.  0 is below every real key.
__device__ __forceinline__ uint64_t route_key(float l, int e) {
    const uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
    const uint32_t k32 = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)k32 << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
    const uint32_t k32 = (uint32_t)(key >> 32);
    const uint32_t u = (k32 & 0x80000000u) ? (k32 & 0x7FFFFFFFu) : ~k32;
    return __uint_as_float(u);
}

// Number of active experts from a permutation's active list, clamped so that a
// corrupt list cannot send a kernel past the arrays it indexes.
__device__ __forceinline__ int active_count(const int32_t* active, int E, int P) {
    const int n = active[0];
    const int cap = E < P ? E : P;
    return n < 0 ? 0 : (n > cap ? cap : n);
}

// Sorted-row range [row0, row0 + n) of expert e; false if out of range.
__device__ __forceinline__ bool expert_rows(const int32_t* offsets, int e, int E, int P, int& row0, int& n) {
    if ((unsigned)e >= (unsigned)E) return false;
    row0 = offsets[e];
    const int end = offsets[e + 1];
    n = end - row0;
    return row0 >= 0 && end <= P && n >= 0;
}

// Exclusive scan of one int per thread over the whole block (blockDim.x a
// multiple of 64, at most 1024); *total receives the sum.  tmp: >= 32 ints of LDS.
__device__ inline int block_exclusive_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int s = lane < (int)(blockDim.x >> 6) ? tmp[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(s, o, WAVE);
            if (lane >= o) s += y;
        }
        if (lane < 16) tmp[16 + lane] = s;
    }
    __syncthreads();
    const int base = wid > 0 ? tmp[16 + wid - 1] : 0;
    *total = tmp[16 + (int)(blockDim.x >> 6) - 1];
    __syncthreads();
    return base + x - v;
}

}  // namespace ds4
