// mfma_f32.hpp -- float32 MFMA tiles fed from LDS (v_mfma_f32_32x32x2f32).
#pragma once
#include <hip/hip_runtime.h>

namespace gds {

typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16x16x4 step: lane (16 g + n16) gives A[n16][g] and B[g][n16]; the result
// holds rows 4 g .. 4 g + 3 of column n16.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 32x32x2 step: lane (32 kg + l32) gives A[l32][kg] and B[kg][l32].
__device__ __forceinline__ f32x16 mfma2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// c + the product of STEPS MFMA steps; A(s) and B(s) give the lane's operands
// of step s.  Each step's operands are loaded two steps ahead of its MFMA and
// sched_barrier pins that order: left alone, the compiler waits for each LDS
// read right before its MFMA, and with one wave per SIMD nothing hides that
// latency.
template <int STEPS, class FA, class FB>
__device__ __forceinline__ f32x16 chain(FA A, FB B, f32x16 c) {
    float a0 = A(0), b0 = B(0);
    float a1 = STEPS > 1 ? A(1) : 0.f, b1 = STEPS > 1 ? B(1) : 0.f;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        float a2 = 0.f, b2 = 0.f;
        if (s + 2 < STEPS) {
            a2 = A(s + 2);
            b2 = B(s + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        c = mfma2(a0, b0, c);
        __builtin_amdgcn_sched_barrier(0);
        a0 = a1;
        b0 = b1;
        a1 = a2;
        b1 = b2;
    }
    return c;
}

}  // namespace gds
