// mfma_f32.hpp -- float32 products on the MFMA units, fed from LDS: on the
// float32 MFMA (v_mfma_f32_32x32x2f32), or in split bf16 on the bf16 MFMA.
#pragma once
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace gds {

typedef float f32x16 __attribute__((ext_vector_type(16)));

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

typedef float f32x8 __attribute__((ext_vector_type(8)));

// hi + lo parts of 8 floats in bf16: hi = RNE(x), lo = RNE(x - hi).  The
// product of two split operands as hi*hi + hi*lo + lo*hi misses the lo*lo term
// and the rounding of each lo, both within about 2^-17 of the product.
__device__ __forceinline__ void split_bf16(const f32x8& x, bf16x8& hi, bf16x8& lo) {
    hi = __builtin_convertvector(x, bf16x8);
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8), bf16x8);
}

// The product of chain<STEPS> (STEPS a multiple of 8) in split bf16 on the
// bf16 MFMA (v_mfma_f32_32x32x16_bf16, 8 times the k of a float32 step in half
// its cycles): a lane's operands of steps 8i .. 8i+7 make its eight values of
// one 32x32x16 step.  Which k a value stands for does not matter as long as A
// and B agree, so A(s) and B(s) are the same accessors as for chain.  A group's
// operands are read one group ahead of its products.
// AX / BX: the A / B operands are bf16 values exactly (inputs given in bf16,
// read before any scaling), so their lo parts are zero: the product then needs
// two MFMAs (one if both are exact) and no lo conversion for that side.
template <int STEPS, bool AX = false, bool BX = false, class FA, class FB>
__device__ __forceinline__ f32x16 chain_split(FA A, FB B, f32x16 c) {
    static_assert(STEPS % 8 == 0, "groups of eight steps");
    constexpr int G = STEPS / 8;
    f32x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = A(j);
        b[j] = B(j);
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
        f32x8 an = a, bn = b;
        if (i + 1 < G) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                an[j] = A(8 * (i + 1) + j);
                bn[j] = B(8 * (i + 1) + j);
            }
        }
        bf16x8 ah, al, bh, bl;
        if constexpr (AX)
            ah = __builtin_convertvector(a, bf16x8);
        else
            split_bf16(a, ah, al);
        if constexpr (BX)
            bh = __builtin_convertvector(b, bf16x8);
        else
            split_bf16(b, bh, bl);
        __builtin_amdgcn_sched_barrier(0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
        if constexpr (!BX) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
        if constexpr (!AX) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        a = an;
        b = bn;
    }
    return c;
}

// chain in float32 or, with SPLIT and whole groups of eight steps, in split bf16
// (AX, BX as for chain_split; they hold only where SPLIT does: bf16 inputs).
template <bool SPLIT, int STEPS, bool AX = false, bool BX = false, class FA, class FB>
__device__ __forceinline__ f32x16 chain_t(FA A, FB B, f32x16 c) {
    if constexpr (SPLIT && STEPS % 8 == 0)
        return chain_split<STEPS, AX, BX>(A, B, c);
    else
        return chain<STEPS>(A, B, c);
}

// chain_t over 8 G steps with the operands fetched a group at a time: A(i) and
// B(i) give the lane's operands of steps 8 i .. 8 i + 7 as one f32x8, so an
// operand laid out along k can come in two 16-byte LDS reads (with the usual
// choice k = 16 i + 8 kg + j for step 8 i + j of lane half kg).  Group i + 1 is
// read before group i's products.  AX / BX as for chain_split.
template <bool SPLIT, int G, bool AX = false, bool BX = false, class FA, class FB>
__device__ __forceinline__ f32x16 chain8_t(FA A, FB B, f32x16 c) {
    f32x8 a = A(0), b = B(0);
#pragma unroll
    for (int i = 0; i < G; ++i) {
        f32x8 an = a, bn = b;
        if (i + 1 < G) {
            an = A(i + 1);
            bn = B(i + 1);
        }
        if constexpr (SPLIT) {
            bf16x8 ah, al, bh, bl;
            if constexpr (AX)
                ah = __builtin_convertvector(a, bf16x8);
            else
                split_bf16(a, ah, al);
            if constexpr (BX)
                bh = __builtin_convertvector(b, bf16x8);
            else
                split_bf16(b, bh, bl);
            __builtin_amdgcn_sched_barrier(0);
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
            if constexpr (!BX) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
            if constexpr (!AX) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; ++j) c = mfma2(a[j], b[j], c);
            __builtin_amdgcn_sched_barrier(0);
        }
        a = an;
        b = bn;
    }
    return c;
}

// Eight floats from 16-byte aligned LDS as two 16-byte reads.
__device__ __forceinline__ f32x8 lds_f32x8(const float* p) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Eight floats down a column: p[0], p[ld], .., p[7 ld].
template <int LD>
__device__ __forceinline__ f32x8 lds_col8(const float* p) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = p[j * LD];
    return r;
}

}  // namespace gds
