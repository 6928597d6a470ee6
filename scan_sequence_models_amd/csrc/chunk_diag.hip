// chunk_diag.hip -- chunkwise scan with diagonal (per-key-channel) gates, float32.
//
// The prefix-scan notes ("Sequential Parallel Duality in Prefix Scannable
// Models", papernotes.org, key design 2) list the diagonal gate among the forms
// of E_t.  Two members, with a_t one decay per key channel:
//
//   gated delta rule:        E_t = diag(a_t) (I - beta_t k_t k_t^T),  f_t = beta_t v_t k_t^T
//   gated linear attention:  E_t = diag(a_t),                         f_t = v_t k_t^T
//
// Inside a chunk (rows = tokens; g_t = cumulative ln a per channel, so
// gamma_t = e^{g_t} <= 1; S the state entering the chunk), unrolling
// S_t = S_{t-1} diag(a_t) + u_t k_t^T with u_t = beta_t (v_t - S_{t-1} diag(a_t) k_t)
// gives the same UT form as the scalar gate, with the decay moved inside the
// channel sums:
//
//   A_ts = beta_t sum_i k_ti k_si e^{g_ti - g_si}   (s < t),   T = (I + A)^-1
//   W    = T diag(beta) (K * gamma),   U = T diag(beta) V - W S^T      (GLA: U = V)
//   P_ts = sum_i q_ti k_si e^{g_ti - g_si}           (s <= t)
//   O    = (Q * gamma) S^T + P U
//   S   <- S diag(gamma_C) + U^T (K * e^{g_C - g})
//
// Every exponent is a difference g_t - g_s with t >= s (or g_C - g_t), so every
// factor is in (0, 1].  The per-channel factors of A and P are evaluated pair by
// pair (one exp2 per token pair and channel); with 32-token chunks that is
// 2 exp2 per token and channel, the dominant cost of this float32 kernel.
//
// One workgroup owns one head and a slice of up to 64 value rows of the state,
// walking the chunks in order with the slice in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;
constexpr int kC = 32;                 // tokens per chunk inside this kernel

template <int MODE, int DK, int SL, typename E>
__global__ __launch_bounds__(kThreads) void chunk_diag_kernel(
    int T, int dv, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    E* __restrict__ o, float* __restrict__ ST) {
    constexpr bool GDN = MODE == 0;
    __shared__ float Qs[kC * DK];   // q, then q * gamma
    __shared__ float Ks[kC * DK];   // k
    __shared__ float Gs[kC * DK];   // g (log2 units: cumulative log2 a)
    __shared__ float Ws[GDN ? kC * DK : 1];
    __shared__ float Us[kC * SL];   // v slice, then U
    __shared__ float Am[kC * kC];   // A (strictly lower)
    __shared__ float Pm[kC * kC];   // P (lower, inclusive)
    __shared__ float Ss[SL * DK];   // state slice, rows r0 .. r0+SL
    __shared__ float bet[kC];

    const int slices = dv / SL;
    const int bh = blockIdx.x / slices;
    const int r0 = (blockIdx.x - bh * slices) * SL;
    const int tid = threadIdx.x;
    const size_t qk_base = (size_t)bh * T * DK;
    const size_t v_base = (size_t)bh * T * dv;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;

    for (int x = tid; x < SL * DK; x += kThreads) Ss[x] = S0 ? S0[s_base + x] : 0.f;

    const int nchunks = (T + kC - 1) / kC;
    for (int n = 0; n < nchunks; ++n) {
        const int c0 = n * kC;
        __syncthreads();  // previous chunk done with every tile
        for (int x = tid; x < kC * DK; x += kThreads) {
            const int t = x / DK;
            const bool in = c0 + t < T;  // past T: identity tokens (a = 1, beta = 0, q = k = v = 0)
            const size_t gi = qk_base + (size_t)c0 * DK + x;
            Qs[x] = in ? io<E>::load(q, gi) : 0.f;
            Ks[x] = in ? io<E>::load(k, gi) : 0.f;
            Gs[x] = in ? __log2f(alpha[gi]) : 0.f;
        }
        for (int x = tid; x < kC * SL; x += kThreads) {
            const int t = x / SL, i = x - t * SL;
            Us[x] = c0 + t < T ? io<E>::load(v, v_base + (size_t)(c0 + t) * dv + r0 + i) : 0.f;
        }
        if (tid < kC) bet[tid] = (GDN && c0 + tid < T) ? beta[(size_t)bh * T + c0 + tid] : 0.f;
        __syncthreads();
        // cumulative log2 decay per channel along the chunk
        for (int c = tid; c < DK; c += kThreads) {
            float run = 0.f;
            for (int t = 0; t < kC; ++t) {
                run += Gs[t * DK + c];
                Gs[t * DK + c] = run;
            }
        }
        __syncthreads();
        // decayed Gram (A) and scores (P), pair by pair
        for (int x = tid; x < kC * kC; x += kThreads) {
            const int t = x / kC, s = x - t * kC;
            float pa = 0.f, pp = 0.f;
            if (s <= t) {
                for (int c = 0; c < DK; ++c) {
                    const float e = exp2f(Gs[t * DK + c] - Gs[s * DK + c]);
                    const float ke = Ks[s * DK + c] * e;
                    pa += Ks[t * DK + c] * ke;
                    pp += Qs[t * DK + c] * ke;
                }
            }
            Am[x] = (GDN && s < t) ? bet[t] * pa : 0.f;
            Pm[x] = pp;
        }
        __syncthreads();
        if constexpr (GDN) {
            // right-hand sides: W = beta (K * gamma), U~ = beta V
            for (int x = tid; x < kC * DK; x += kThreads) {
                const int t = x / DK;
                Ws[x] = bet[t] * Ks[x] * exp2f(Gs[x]);
            }
            for (int x = tid; x < kC * SL; x += kThreads) Us[x] *= bet[x / SL];
            __syncthreads();
            // forward substitution: row i of [W | U~] -= sum_{j<i} A_ij row j
            for (int i = 1; i < kC; ++i) {
                for (int c = tid; c < DK + SL; c += kThreads) {
                    if (c < DK) {
                        float acc = Ws[i * DK + c];
                        for (int j = 0; j < i; ++j) acc -= Am[i * kC + j] * Ws[j * DK + c];
                        Ws[i * DK + c] = acc;
                    } else {
                        const int cc = c - DK;
                        float acc = Us[i * SL + cc];
                        for (int j = 0; j < i; ++j) acc -= Am[i * kC + j] * Us[j * SL + cc];
                        Us[i * SL + cc] = acc;
                    }
                }
                __syncthreads();
            }
            // U = U~ - W S^T
            for (int x = tid; x < kC * SL; x += kThreads) {
                const int t = x / SL, i = x - t * SL;
                float acc = Us[x];
                for (int j = 0; j < DK; ++j) acc -= Ws[t * DK + j] * Ss[i * DK + j];
                Us[x] = acc;
            }
            __syncthreads();
        }
        // Q * gamma (in place)
        for (int x = tid; x < kC * DK; x += kThreads) Qs[x] *= exp2f(Gs[x]);
        __syncthreads();
        // O = (Q * gamma) S^T + P U
        for (int x = tid; x < kC * SL; x += kThreads) {
            const int t = x / SL, i = x - t * SL;
            if (c0 + t < T) {
                float acc = 0.f;
                for (int j = 0; j < DK; ++j) acc += Qs[t * DK + j] * Ss[i * DK + j];
                for (int s = 0; s <= t; ++s) acc += Pm[t * kC + s] * Us[s * SL + i];
                io<E>::store(o, v_base + (size_t)(c0 + t) * dv + r0 + i, acc);
            }
        }
        // K * e^{g_C - g} (in place: Ks is not read by the read-out)
        for (int x = tid; x < kC * DK; x += kThreads) {
            const int c = x % DK;
            Ks[x] *= exp2f(Gs[(kC - 1) * DK + c] - Gs[x]);
        }
        __syncthreads();
        // S <- S diag(gamma_C) + U^T (K * e^{g_C - g})
        for (int x = tid; x < SL * DK; x += kThreads) {
            const int i = x / DK, j = x - i * DK;
            float acc = Ss[x] * exp2f(Gs[(kC - 1) * DK + j]);
            for (int t = 0; t < kC; ++t) acc += Us[t * SL + i] * Ks[t * DK + j];
            Ss[x] = acc;
        }
    }
    __syncthreads();
    if (ST)
        for (int x = tid; x < SL * DK; x += kThreads) ST[s_base + x] = Ss[x];
}

template <int MODE, int DK, typename E>
hipError_t launch_dk(int BH, int T, int dv, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* S0, void* o, float* ST,
                     hipStream_t s) {
    const E* qq = static_cast<const E*>(q);
    const E* kk = static_cast<const E*>(k);
    const E* vv = static_cast<const E*>(v);
    E* oo = static_cast<E*>(o);
    if (dv % 64 == 0) {
        hipLaunchKernelGGL((chunk_diag_kernel<MODE, DK, 64, E>), dim3((unsigned)((size_t)BH * (dv / 64))),
                           dim3(kThreads), 0, s, T, dv, qq, kk, vv, alpha, beta, S0, oo, ST);
    } else {
        hipLaunchKernelGGL((chunk_diag_kernel<MODE, DK, 16, E>), dim3((unsigned)((size_t)BH * (dv / 16))),
                           dim3(kThreads), 0, s, T, dv, qq, kk, vv, alpha, beta, S0, oo, ST);
    }
    return hipGetLastError();
}

template <int MODE, typename E>
hipError_t launch_mode(int BH, int T, int dk, int dv, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const float* S0, void* o, float* ST,
                       hipStream_t s) {
    switch (dk) {
        case 16: return launch_dk<MODE, 16, E>(BH, T, dv, q, k, v, alpha, beta, S0, o, ST, s);
        case 32: return launch_dk<MODE, 32, E>(BH, T, dv, q, k, v, alpha, beta, S0, o, ST, s);
        case 64: return launch_dk<MODE, 64, E>(BH, T, dv, q, k, v, alpha, beta, S0, o, ST, s);
        case 128: return launch_dk<MODE, 128, E>(BH, T, dv, q, k, v, alpha, beta, S0, o, ST, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool chunk_diag_supported(int dk, int dv) {
    const bool dk_ok = dk == 16 || dk == 32 || dk == 64 || dk == 128;
    return dk_ok && dv >= 16 && dv % 16 == 0 && dv <= 4096;
}

hipError_t launch_chunk_diag(int mode, int dtype, int BH, int T, int dk, int dv, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta,
                             const float* S0, void* o, float* ST, hipStream_t s) {
    if (dtype == 0)
        return mode == 0 ? launch_mode<0, float>(BH, T, dk, dv, q, k, v, alpha, beta, S0, o, ST, s)
                         : launch_mode<1, float>(BH, T, dk, dv, q, k, v, alpha, beta, S0, o, ST, s);
    return mode == 0 ? launch_mode<0, uint16_t>(BH, T, dk, dv, q, k, v, alpha, beta, S0, o, ST, s)
                     : launch_mode<1, uint16_t>(BH, T, dk, dv, q, k, v, alpha, beta, S0, o, ST, s);
}

}  // namespace gds
