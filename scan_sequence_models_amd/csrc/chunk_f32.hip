// chunk_f32.hip -- float32 chunkwise scan (any supported size; the precise path).
//
// The prefix-scan notes ("Sequential Parallel Duality in Prefix Scannable
// Models", papernotes.org, overall framework) cut the sequence into chunks,
// encode each chunk, carry the state across chunk boundaries and read every
// chunk out from its exclusive prefix state.  For the affine monoid of the
// gated delta rule the chunk of C tokens (rows; g = in-chunk cumulative
// log-decay, gamma = exp(g)) obeys, with S the state entering the chunk:
//
//   A  = strict_lower( diag(beta) (Gamma * K K^T) ),  Gamma_ij = exp(g_i - g_j)
//   (I + A) [W | U~] = [diag(beta gamma) K | diag(beta_w) V]  (forward substitution)
//   U  = U~ - W S^T
//   O  = diag(gamma) Q S^T + (Q K^T * Gamma * M) U            (M: inclusive causal)
//   S <- gamma_C S + U^T diag(exp(g_C - g)) K
//
// and for gated linear attention U = V (no A, no W).  These follow from
// unrolling the token recurrence S_t = alpha_t S_{t-1} + u_t k_t^T with
// u_t = beta_w,t v_t - beta_t alpha_t S_{t-1} k_t inside one chunk (beta_w, the
// write strength, equals beta except where erase and write are split).  Decay ratios are
// always exp(g_i - g_j) with i >= j (never quotients of products), so they stay
// in (0, 1].
//
// One workgroup owns one head and a slice of kSlice value rows of its state and
// walks the chunks in order with the state slice resident in LDS.  Every step
// is plain float32 FMA arithmetic over LDS tiles: this kernel exists for exact
// float32 parity, not for speed (the bf16 MFMA kernel is the fast path).
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 16;  // value rows of S per workgroup

template <int MODE, int DK, int C, typename E>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(
    int T, int dv, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ beta_w, const float* __restrict__ S0, E* __restrict__ o,
    float* __restrict__ ST) {
    constexpr bool GDN = MODE == 0;
    __shared__ float Qs[C * DK];
    __shared__ float Ks[C * DK];
    __shared__ float Ws[GDN ? C * DK : 1];
    __shared__ float Vs[C * kSlice];
    __shared__ float Us[C * kSlice];
    __shared__ float AP[C * C];
    __shared__ float Ss[kSlice * DK];
    __shared__ float g[C], gam[C], bet[C], bw[C], dec[C];

    const int slices = dv / kSlice;
    const int bh = blockIdx.x / slices;
    const int r0 = (blockIdx.x - bh * slices) * kSlice;
    const int tid = threadIdx.x;
    const size_t qk_base = (size_t)bh * T * DK;
    const size_t v_base = (size_t)bh * T * dv;
    const size_t a_base = (size_t)bh * T;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;

    for (int x = tid; x < kSlice * DK; x += kThreads) Ss[x] = S0 ? S0[s_base + x] : 0.f;

    const int nchunks = (T + C - 1) / C;
    for (int n = 0; n < nchunks; ++n) {
        const int c0 = n * C;
        __syncthreads();  // previous chunk finished with every tile
        for (int x = tid; x < C * DK; x += kThreads) {
            const int t = x / DK, j = x - (x / DK) * DK;
            const bool in = c0 + t < T;
            Qs[x] = in ? io<E>::load(q, qk_base + (size_t)(c0 + t) * DK + j) : 0.f;
            Ks[x] = in ? io<E>::load(k, qk_base + (size_t)(c0 + t) * DK + j) : 0.f;
        }
        for (int x = tid; x < C * kSlice; x += kThreads) {
            const int t = x / kSlice, i = x - t * kSlice;
            Vs[x] = c0 + t < T ? io<E>::load(v, v_base + (size_t)(c0 + t) * dv + r0 + i) : 0.f;
        }
        if (tid < C) {
            const bool in = c0 + tid < T;  // padded tokens: alpha = 1, beta = 0
            g[tid] = in ? logf(alpha[a_base + c0 + tid]) : 0.f;
            bet[tid] = (GDN && in) ? beta[a_base + c0 + tid] : 0.f;
            bw[tid] = (GDN && in) ? beta_w[a_base + c0 + tid] : 0.f;
        }
        __syncthreads();
        if (tid == 0) {
            float run = 0.f;
            for (int t = 0; t < C; ++t) { run += g[t]; g[t] = run; }
        }
        __syncthreads();
        if (tid < C) {
            gam[tid] = expf(g[tid]);
            dec[tid] = expf(g[C - 1] - g[tid]);
        }
        __syncthreads();

        const float* U = Vs;  // gla: U = V
        if constexpr (GDN) {
            for (int x = tid; x < C * C; x += kThreads) {
                const int i = x / C, j = x - (x / C) * C;
                float a = 0.f;
                if (i > j) {
                    for (int d = 0; d < DK; ++d) a += Ks[i * DK + d] * Ks[j * DK + d];
                    a *= bet[i] * expf(g[i] - g[j]);
                }
                AP[x] = a;
            }
            for (int x = tid; x < C * DK; x += kThreads) {
                const int t = x / DK;
                Ws[x] = bet[t] * gam[t] * Ks[x];
            }
            for (int x = tid; x < C * kSlice; x += kThreads) {
                const int t = x / kSlice;
                Us[x] = bw[t] * Vs[x];
            }
            __syncthreads();
            // forward substitution: row i of [W | U~] -= sum_{j<i} A_ij row j
            for (int i = 1; i < C; ++i) {
                for (int c = tid; c < DK + kSlice; c += kThreads) {
                    if (c < DK) {
                        float acc = Ws[i * DK + c];
                        for (int j = 0; j < i; ++j) acc -= AP[i * C + j] * Ws[j * DK + c];
                        Ws[i * DK + c] = acc;
                    } else {
                        const int cc = c - DK;
                        float acc = Us[i * kSlice + cc];
                        for (int j = 0; j < i; ++j) acc -= AP[i * C + j] * Us[j * kSlice + cc];
                        Us[i * kSlice + cc] = acc;
                    }
                }
                __syncthreads();
            }
            // U = U~ - W S^T
            for (int x = tid; x < C * kSlice; x += kThreads) {
                const int t = x / kSlice, i = x - t * kSlice;
                float acc = Us[x];
                for (int j = 0; j < DK; ++j) acc -= Ws[t * DK + j] * Ss[i * DK + j];
                Us[x] = acc;
            }
            U = Us;
            __syncthreads();
        }
        // P = Q K^T * Gamma, inclusive causal mask
        for (int x = tid; x < C * C; x += kThreads) {
            const int t = x / C, s = x - (x / C) * C;
            float p = 0.f;
            if (s <= t) {
                for (int d = 0; d < DK; ++d) p += Qs[t * DK + d] * Ks[s * DK + d];
                p *= expf(g[t] - g[s]);
            }
            AP[x] = p;
        }
        __syncthreads();
        // O = diag(gamma) Q S^T + P U
        for (int x = tid; x < C * kSlice; x += kThreads) {
            const int t = x / kSlice, i = x - t * kSlice;
            if (c0 + t < T) {
                float qs = 0.f;
                for (int j = 0; j < DK; ++j) qs += Qs[t * DK + j] * Ss[i * DK + j];
                float pu = 0.f;
                for (int s = 0; s <= t; ++s) pu += AP[t * C + s] * U[s * kSlice + i];
                io<E>::store(o, v_base + (size_t)(c0 + t) * dv + r0 + i, gam[t] * qs + pu);
            }
        }
        __syncthreads();
        // S <- gamma_C S + U^T diag(dec) K
        for (int x = tid; x < kSlice * DK; x += kThreads) {
            const int i = x / DK, j = x - (x / DK) * DK;
            float acc = gam[C - 1] * Ss[x];
            for (int t = 0; t < C; ++t) acc += U[t * kSlice + i] * dec[t] * Ks[t * DK + j];
            Ss[x] = acc;
        }
    }
    __syncthreads();
    if (ST)
        for (int x = tid; x < kSlice * DK; x += kThreads) ST[s_base + x] = Ss[x];
}

template <int MODE, int DK, int C, typename E>
hipError_t launch3(int BH, int T, int dv, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* bw, const float* S0, void* o, float* ST,
                   hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)BH * (dv / kSlice)));
    hipLaunchKernelGGL((chunk_f32_kernel<MODE, DK, C, E>), grid, dim3(kThreads), 0, stream, T, dv,
                       static_cast<const E*>(q), static_cast<const E*>(k),
                       static_cast<const E*>(v), alpha, beta, bw, S0, static_cast<E*>(o), ST);
    return hipGetLastError();
}

template <int MODE, int DK, typename E>
hipError_t launch2(int chunk, int BH, int T, int dv, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* bw, const float* S0, void* o, float* ST,
                   hipStream_t s) {
    switch (chunk) {
        case 16: return launch3<MODE, DK, 16, E>(BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        case 32: return launch3<MODE, DK, 32, E>(BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        case 64: return launch3<MODE, DK, 64, E>(BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        default: return hipErrorInvalidValue;
    }
}

template <int MODE, typename E>
hipError_t launch1(int dk, int chunk, int BH, int T, int dv, const void* q, const void* k,
                   const void* v, const float* alpha, const float* beta, const float* bw, const float* S0,
                   void* o, float* ST, hipStream_t s) {
    switch (dk) {
        case 16: return launch2<MODE, 16, E>(chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        case 32: return launch2<MODE, 32, E>(chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        case 64: return launch2<MODE, 64, E>(chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        case 128: return launch2<MODE, 128, E>(chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool chunk_f32_supported(int mode, int dk, int dv, int chunk) {
    (void)mode;
    const bool dk_ok = dk == 16 || dk == 32 || dk == 64 || dk == 128;
    const bool c_ok = chunk == 16 || chunk == 32 || chunk == 64;
    return dk_ok && c_ok && dv >= kSlice && dv % kSlice == 0 && dv <= 4096;
}

hipError_t launch_chunk_f32(int mode, int dtype, int BH, int T, int dk, int dv, int chunk,
                            const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* bw, const float* S0, void* o, float* ST,
                            hipStream_t s) {
    if (dtype == 0) {
        if (mode == 0) return launch1<0, float>(dk, chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
        return launch1<1, float>(dk, chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
    }
    if (mode == 0) return launch1<0, uint16_t>(dk, chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
    return launch1<1, uint16_t>(dk, chunk, BH, T, dv, q, k, v, alpha, beta, bw, S0, o, ST, s);
}

}  // namespace gds
