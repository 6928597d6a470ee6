// solve.hpp -- the unit lower triangular inverse of a chunk's 32x32 UT
// transform, on one wave.
#pragma once
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_f32.hpp"

namespace gds {

// T = (I + diag(bet) B)^-1 for the strictly lower part of the 32x32 matrix B
// (row stride LB, 16-byte rows) into Tm (row stride LT), from its 16x16
// blocks: the two diagonal blocks D0, D1 by forward substitution side by side
// (lane (b, c) of each half-wave owns column c of block b,
// x_r = [r == c] - bet_r sum_{j<r} B_rj x_j, rows read as float4 two rows
// ahead), then T10 = -D1 diag(bet) B10 D0 on the fp32 MFMA (16x16x4).  The
// upper right block of Tm is not written: it stays zero from the start.  All
// 64 lanes of the wave take part.
template <int LB, int LT>
__device__ __forceinline__ void solve_unit_lower(const float* Bm, const float* bet, float* Tm, int lane) {
    const int b = (lane >> 4) & 1, c = lane & 15, kg = lane >> 5;
    const float* Bb = Bm + 16 * b * LB + 16 * b;
    float br[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) br[r] = bet[16 * b + r];
    f32x4 rw[3][4];  // rows r, r + 1, r + 2 in flight
    auto load_row = [&](int r, f32x4 (&dst)[4]) {
#pragma unroll
        for (int q = 0; q < (r + 3) / 4; ++q) dst[q] = *reinterpret_cast<const f32x4*>(&Bb[r * LB + 4 * q]);
    };
    load_row(1, rw[1]);
    load_row(2, rw[2]);
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r + 2 < 16) load_row(r + 2, rw[(r + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int q = 0; q < (r + 3) / 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * q + i;
                if (j < r) {
                    if (i & 1) s1 += rw[r % 3][q][i] * x[j];
                    else s0 += rw[r % 3][q][i] * x[j];
                }
            }
        x[r] = (r == c ? 1.f : 0.f) - br[r] * (s0 + s1);
    }
    if (kg == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(16 * b + r) * LT + 16 * b + c] = x[r];
    }
    // T10 = -D1 (diag(bet) B10) D0: lane (n16, g4) supplies contraction indices
    // 4 g4 .. 4 g4 + 3 and holds rows 4 g4 .. 4 g4 + 3 of column n16
    const int n16 = lane & 15, g4 = lane >> 4;
    f32x4 y = {}, t10 = {};
    const f32x4 br10 = *reinterpret_cast<const f32x4*>(&Bm[(16 + n16) * LB + 4 * g4]);
    const float bs = bet[16 + n16];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) y = mfma4(br10[kk] * bs, Tm[(4 * g4 + kk) * LT + n16], y);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t10 = mfma4(Tm[(16 + n16) * LT + 16 + 4 * g4 + kk], y[kk], t10);
#pragma unroll
    for (int r = 0; r < 4; ++r) Tm[(16 + 4 * g4 + r) * LT + n16] = -t10[r];
}

}  // namespace gds
