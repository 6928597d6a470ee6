// common.hpp -- small device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gds {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 <-> float32.  Widening is exact; narrowing rounds to nearest even
// (gfx950 converts in hardware).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// Element access for the two I/O types (float and bfloat16 stored as uint16_t).
template <typename T> struct io;
template <> struct io<float> {
    __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
    __device__ static __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
    // four consecutive elements starting at i (i multiple of 4, 16-byte aligned base)
    __device__ static __forceinline__ float4 load4(const float* p, size_t i) {
        return *reinterpret_cast<const float4*>(p + i);
    }
};
template <> struct io<uint16_t> {
    __device__ static __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ static __forceinline__ void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
    __device__ static __forceinline__ float4 load4(const uint16_t* p, size_t i) {
        uint2 u = *reinterpret_cast<const uint2*>(p + i);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
};

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

}  // namespace gds
