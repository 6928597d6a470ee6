// decode.hip -- single-token state update, one streaming pass over each state.
//
// Sequential (inference) view of the affine scan: one update of the fixed-size
// state per token ("Sequential Parallel Duality in Prefix Scannable Models",
// papernotes.org notes, key design 1; constant-size state, key design 2).  Per
// state S (dv x dk, fp32, in place) and token (q, k, v, alpha, beta):
//
//   (diagonal gates: S <- S diag(a) first, then alpha = 1 below)
//   a = S k,  b = S q                         (row dot products of the old S)
//   gdn: u = beta_w v - beta alpha a      gla: u = v
//   (beta_w, the write strength, is beta unless erase and write are split)
//   S  <- alpha S + u k^T                     (= S E + f for this token)
//   o   = S_new q = alpha b + (k . q) u
//
// The work is HBM-bound (64 KB read + 64 KB written per 128x128 state, ~7 d^2
// flop), so the kernel is organised around the stream: rows of S are
// independent, a row of dk floats is covered by dk/4 lanes with one 16-byte
// load each, and every thread issues all of its row loads before anything
// else; the token's v entries are fetched up front too, the row reductions run
// on DPP lane permutes, and the state is read and written with non-temporal
// loads and stores (each byte is touched once per step).  A workgroup takes 32
// rows (64 for dk = 16): many short workgroups keep the CUs streaming, where
// one 128-row workgroup per state left gaps at each workgroup's start and a
// tail at the end of the grid (measured 107 us per step for 4096 128x128
// states, against 89 us now).
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;
// rows per workgroup: 32, or one pass of the block where that is more (dk = 16)
template <int DK>
constexpr int kRowsPerBlock = (kThreads / (DK / 4)) > 32 ? (kThreads / (DK / 4)) : 32;

template <int DK, int MODE, bool DIAG, typename E>
__global__ __launch_bounds__(kThreads) void decode_kernel(int dv, int row_blocks,
                                                          const E* __restrict__ q,
                                                          const E* __restrict__ k,
                                                          const E* __restrict__ v,
                                                          const float* __restrict__ alpha,
                                                          const float* __restrict__ beta,
                                                          const float* __restrict__ beta_w,
                                                          float* __restrict__ S,
                                                          E* __restrict__ o) {
    constexpr int L = DK / 4;                       // lanes per row
    constexpr int kRowsPerWavePass = kWave / L;
    constexpr int kRowsPerPass = kRowsPerWavePass * (kThreads / kWave);
    constexpr int kPasses = kRowsPerBlock<DK> / kRowsPerPass;

    const int n = blockIdx.x / row_blocks;
    const int rb = blockIdx.x - n * row_blocks;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int sub = lane % L;
    const int rsub = lane / L;

    // The state rows first: every load of the block is in flight before any
    // other memory operation.  Rows past dv (dv not a multiple of the block)
    // are clamped to a valid row; their results are not stored.
    f32x4* Sn = reinterpret_cast<f32x4*>(S + (size_t)n * dv * DK);
    int rows[kPasses];
    f32x4 s[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        rows[p] = rb * kRowsPerBlock<DK> + p * kRowsPerPass + wave * kRowsPerWavePass + rsub;
        const int rc = rows[p] < dv ? rows[p] : dv - 1;
        s[p] = __builtin_nontemporal_load(Sn + (size_t)rc * (DK / 4) + sub);
    }
    const float4 k4 = io<E>::load4(k, (size_t)n * DK + sub * 4);
    const float4 q4 = io<E>::load4(q, (size_t)n * DK + sub * 4);
    const float al = DIAG ? 1.f : alpha[n];
    const float be = MODE == 0 ? beta[n] : 0.f;
    const float bw = MODE == 0 ? beta_w[n] : 0.f;
    float vr[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        vr[p] = io<E>::load(v, (size_t)n * dv + (rows[p] < dv ? rows[p] : dv - 1));
    const float kq = group_sum<L>(k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w);
    if constexpr (DIAG) {  // per-key-channel decay of the state before the update reads it
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(alpha + (size_t)n * DK + sub * 4);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) s[p] *= a4;
    }

#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float a = s[p].x * k4.x + s[p].y * k4.y + s[p].z * k4.z + s[p].w * k4.w;
        float b = s[p].x * q4.x + s[p].y * q4.y + s[p].z * q4.z + s[p].w * q4.w;
        a = group_sum<L>(a);
        b = group_sum<L>(b);
        const float u = MODE == 0 ? bw * vr[p] - be * (al * a) : vr[p];
        f32x4 r;
        r.x = al * s[p].x + u * k4.x;
        r.y = al * s[p].y + u * k4.y;
        r.z = al * s[p].z + u * k4.z;
        r.w = al * s[p].w + u * k4.w;
        if (rows[p] < dv) {
            __builtin_nontemporal_store(r, Sn + (size_t)rows[p] * (DK / 4) + sub);
            if (sub == 0) io<E>::store(o, (size_t)n * dv + rows[p], al * b + kq * u);
        }
    }
}

template <int DK, typename E>
hipError_t launch_typed(int mode, int N, int dv, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const float* beta_w, float* S, void* o,
                        hipStream_t stream) {
    // mode: 0 gated delta rule, 1 gated linear attention, 2 and 3 the same with
    // diagonal gates (alpha holds dk decays per state)
    const int rb = (dv + kRowsPerBlock<DK> - 1) / kRowsPerBlock<DK>;
    const dim3 grid((unsigned)((size_t)N * rb));
    const E* qq = static_cast<const E*>(q);
    const E* kk = static_cast<const E*>(k);
    const E* vv = static_cast<const E*>(v);
    E* oo = static_cast<E*>(o);
    if (mode == 0)
        hipLaunchKernelGGL((decode_kernel<DK, 0, false, E>), grid, dim3(kThreads), 0, stream, dv, rb, qq,
                           kk, vv, alpha, beta, beta_w, S, oo);
    else if (mode == 1)
        hipLaunchKernelGGL((decode_kernel<DK, 1, false, E>), grid, dim3(kThreads), 0, stream, dv, rb, qq,
                           kk, vv, alpha, beta, beta_w, S, oo);
    else if (mode == 2)
        hipLaunchKernelGGL((decode_kernel<DK, 0, true, E>), grid, dim3(kThreads), 0, stream, dv, rb, qq,
                           kk, vv, alpha, beta, beta_w, S, oo);
    else
        hipLaunchKernelGGL((decode_kernel<DK, 1, true, E>), grid, dim3(kThreads), 0, stream, dv, rb, qq,
                           kk, vv, alpha, beta, beta_w, S, oo);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_dk(int mode, int N, int dk, int dv, const void* q, const void* k,
                     const void* v, const float* alpha, const float* beta, const float* beta_w, float* S, void* o,
                     hipStream_t stream) {
    switch (dk) {
        case 16: return launch_typed<16, E>(mode, N, dv, q, k, v, alpha, beta, beta_w, S, o, stream);
        case 32: return launch_typed<32, E>(mode, N, dv, q, k, v, alpha, beta, beta_w, S, o, stream);
        case 64: return launch_typed<64, E>(mode, N, dv, q, k, v, alpha, beta, beta_w, S, o, stream);
        case 128: return launch_typed<128, E>(mode, N, dv, q, k, v, alpha, beta, beta_w, S, o, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int dk) { return dk == 16 || dk == 32 || dk == 64 || dk == 128; }

hipError_t launch_decode(int mode, int dtype, int N, int dk, int dv, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const float* beta_w, float* S, void* o, hipStream_t stream) {
    if (dtype == 0)
        return launch_dk<float>(mode, N, dk, dv, q, k, v, alpha, beta, beta_w, S, o, stream);
    return launch_dk<uint16_t>(mode, N, dk, dv, q, k, v, alpha, beta, beta_w, S, o, stream);
}

}  // namespace gds
