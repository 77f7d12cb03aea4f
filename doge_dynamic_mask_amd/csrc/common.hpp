// Device helpers shared by the DMA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Order-preserving map float -> uint32 for the top-w selection: a larger
// float gives a larger key; -0.0 is folded onto +0.0 so that the integer
// order agrees with float comparison (NaN is outside the contract).
__device__ __forceinline__ uint32_t ordkey(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit selection key: dt order in the high word, then the lower index
// first (its complement) in the low word.  Keys of distinct positions differ.
__device__ __forceinline__ uint64_t selkey(float dtv, uint32_t j) {
    return ((uint64_t)ordkey(dtv) << 32) | (uint64_t)(~j);
}
__device__ __forceinline__ uint32_t selkey_idx(uint64_t k) { return ~(uint32_t)k; }

// Kept test of key j (value dtv) against a row threshold pair.
__device__ __forceinline__ bool kept_test(float dtv, int j, float tau, int tie) {
    return (dtv > tau) || (dtv == tau && j <= tie);
}

// Valid length of batch b from a caller's lengths array (NULL: n), clamped
// to [0, n]: the documented range is [1, n], and a value outside it must not
// index past the rows it bounds.
__device__ __forceinline__ int clamp_len(const int32_t *lens, int b, int n) {
    return lens ? min(max(lens[b], 0), n) : n;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Sum / max across the two 32-lane halves of a wave (lanes l and l^32).
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace dma
