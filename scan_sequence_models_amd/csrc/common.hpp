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

// The value of the lane that DPP control word CTRL selects (all rows and banks).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float y) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G consecutive lanes (G in {4, 8, 16, 32, 64});
// every lane of the group receives the group's sum.  Within a 16-lane row the
// partners come from DPP (quad permutes, then the half-row and row mirrors);
// across rows from a 32-lane swizzle and a 64-lane shuffle.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
    x += dpp_move<0xB1>(x);                          // lane ^ 1
    x += dpp_move<0x4E>(x);                          // lane ^ 2
    if constexpr (G >= 8) x += dpp_move<0x141>(x);   // row half mirror: the other quad of the 8
    if constexpr (G >= 16) x += dpp_move<0x140>(x);  // row mirror: the other 8 of the row
    if constexpr (G >= 32)                      // lane ^ 16 within 32 (bit-mode swizzle)
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    if constexpr (G >= 64) x += __shfl_xor(x, 32, kWave);
    return x;
}

// (unit, part) of block x when each unit is split into `parts` blocks: blocks
// are dealt round-robin over the 8 XCDs, so when the unit count is a multiple
// of 8 the parts of a unit are placed on one XCD and share its L2.
__device__ __forceinline__ void unit_part(int x, int units, int parts, int& unit, int& part) {
    if ((units & 7) == 0) {
        const int xcd = x & 7, j = x >> 3;
        unit = (j / parts) * 8 + xcd;
        part = j % parts;
    } else {
        unit = x / parts;
        part = x % parts;
    }
}

}  // namespace gds
