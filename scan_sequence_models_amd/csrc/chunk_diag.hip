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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_f32.hpp"

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

// The same chunk algorithm with its products on the float32 MFMA
// (v_mfma_f32_32x32x2f32, fp32 accuracy) for slices of 64 value rows and
// dk >= 32.  Per chunk:
//   1. q, k, log2 a and the value slice come in; log2 a is summed along the
//      chunk per channel;
//   2. the decayed Gram A and scores P over the 496 strictly lower token pairs
//      (one exp2 per pair and channel, float4 loads along the channels, two
//      pairs per thread sharing token t's loads; the diagonal of P needs no
//      exponential), and the scaled copies q gamma,
//      -beta k gamma and k e^{g_C - g};
//   3. T = (I + A)^-1 by one wave (a lane per column, forward substitution with
//      the rows of A read as float4), beside X = R_v - R_w S^T and the start of
//      O = (Q gamma) S^T on the other three waves;
//   4. U = T X, then O += P U beside the state update
//      S <- S diag(gamma_C) + U^T (K e^{g_C - g}), all as 32x32 tiles.
// U = T (R_v - R_w S^T) is the same product as T R_v - (T R_w) S^T, grouped so
// that the key-long product does not wait for the inverse.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
constexpr int kSL = 64;      // value rows per workgroup
constexpr int kLT = kC + 4;  // row stride of the 32x32 T and P tiles (float4 rows)

template <int MODE, int DK, typename E>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_diag_mfma_kernel(
    int T, int dv, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    E* __restrict__ o, float* __restrict__ ST) {
    constexpr bool GDN = MODE == 0;
    constexpr int NJ = DK / 32;  // 32-column tiles of a key-wide row
    // Row strides.  The Gram reads float4 runs of channels with one token per
    // lane: a stride of DK + 4 keeps those 16-byte loads aligned and spreads
    // eight consecutive lanes over distinct bank groups.  The MFMA operands
    // read one float per lane down a column: an odd stride (DK + 1) puts the
    // 32 lanes into 32 banks.
    constexpr int L4 = DK + 4;
    constexpr int L1 = DK + 1;
    __shared__ __align__(16) float Qs[kC * L4];  // q
    __shared__ __align__(16) float Ks[kC * L4];  // k
    __shared__ __align__(16) float Gs[kC * L4];  // cumulative log2 decay
    __shared__ float Qg[kC * L1];                // q * gamma
    __shared__ float Kt[kC * L1];                // k * e^{g_C - g}
    __shared__ float Rw[GDN ? kC * L1 : 1];      // -beta (k * gamma)
    __shared__ float Us[kC * kSL];               // v slice (GDN: beta v), then U
    __shared__ __align__(16) float Am[GDN ? kC * kC : 1];  // A (strictly lower)
    __shared__ float Tm[GDN ? kC * kLT : 1];
    __shared__ float Pm[kC * kLT];               // P (lower, inclusive; zero above)
    __shared__ float Ss[kSL * L1];               // state slice
    __shared__ float Ob[GDN ? 16 * 64 : 1];      // a partial O tile (accumulator layout)
    __shared__ float bet[kC];

    const int slices = dv / kSL;
    const int bh = blockIdx.x / slices;
    const int r0 = (blockIdx.x - bh * slices) * kSL;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, kg = lane >> 5;
    const size_t qk_base = (size_t)bh * T * DK;
    const size_t v_base = (size_t)bh * T * dv;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;
    // accumulator element e of a 32x32 tile: row 8 (e / 4) + 4 kg + e % 4, column l32
    auto row = [&](int e) { return 8 * (e >> 2) + 4 * kg + (e & 3); };

    for (int x = tid; x < kSL * DK; x += kThreads) Ss[x / DK * L1 + x % DK] = S0 ? S0[s_base + x] : 0.f;
    for (int x = tid; x < kC * kLT; x += kThreads) Pm[x] = 0.f;

    // The next chunk's inputs are fetched into registers while this chunk
    // computes (one wave per SIMD leaves no other way to hide HBM latency).
    // The loads are unconditional, from a token index clamped into the
    // sequence, and keep the raw element; masking and conversion happen when
    // they are written to LDS, so no load waits inside the fetch.
    constexpr int NQ = kC * DK / kThreads;   // key-wide elements per thread and chunk
    constexpr int NV = kC * kSL / kThreads;  // value elements per thread and chunk
    E pq[NQ], pk[NQ], pv[NV];
    float pa[NQ], pb = 0.f;
    auto fetch = [&](int cn) {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int x = tid + m * kThreads, t = min(cn + x / DK, T - 1);
            const size_t gi = qk_base + (size_t)t * DK + x % DK;
            pq[m] = q[gi];
            pk[m] = k[gi];
            pa[m] = alpha[gi];
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreads, t = min(cn + x / kSL, T - 1);
            pv[m] = v[v_base + (size_t)t * dv + r0 + x % kSL];
        }
        if (GDN && tid < kC) pb = beta[(size_t)bh * T + min(cn + tid, T - 1)];
    };
    fetch(0);

    const int nchunks = (T + kC - 1) / kC;
    for (int n = 0; n < nchunks; ++n) {
        const int c0 = n * kC;
        __syncthreads();  // the previous chunk is done with every array
        // past T: identity tokens (a = 1, beta = 0, q = k = v = 0)
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int x = tid + m * kThreads, y = x / DK * L4 + x % DK;
            const bool in = c0 + x / DK < T;
            Qs[y] = in ? to_f32(pq[m]) : 0.f;
            Ks[y] = in ? to_f32(pk[m]) : 0.f;
            Gs[y] = in ? __log2f(pa[m]) : 0.f;
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreads;
            Us[x] = c0 + x / kSL < T ? to_f32(pv[m]) : 0.f;
        }
        if (tid < kC) bet[tid] = c0 + tid < T ? pb : 0.f;
        if (n + 1 < nchunks) fetch(c0 + kC);
        __syncthreads();
        if constexpr (GDN)
            for (int x = tid; x < kC * kSL; x += kThreads) Us[x] *= bet[x / kSL];
        for (int c = tid; c < DK; c += kThreads) {
            float run = 0.f;
#pragma unroll 8
            for (int t = 0; t < kC; ++t) {
                run += Gs[t * L4 + c];
                Gs[t * L4 + c] = run;
            }
        }
        __syncthreads();
        // decayed Gram and scores over the strictly lower pairs s < t, two pairs (t, 2b) and
        // (t, 2b + 1) per thread so that they share the loads of token t: row t holds
        // ceil(t / 2) such blocks, floor(t^2 / 4) of them precede it, and rows 1 .. 31 hold
        // exactly 256, one per thread (the second pair of the last block of an odd row is the
        // diagonal, which is not stored here)
        {
            static_assert(kC == 32 && kThreads == 256, "one Gram block per thread");
            const int p = tid;
            int t = (int)__builtin_sqrtf(4.f * (float)p + 1.f);
            if ((t * t) / 4 > p) --t;
            if (((t + 1) * (t + 1)) / 4 <= p) ++t;
            const int s1 = 2 * (p - (t * t) / 4), s2 = s1 + 1;
            const float4* gt = reinterpret_cast<const float4*>(Gs + t * L4);
            const float4* kt = reinterpret_cast<const float4*>(Ks + t * L4);
            const float4* qt = reinterpret_cast<const float4*>(Qs + t * L4);
            const float4* g1p = reinterpret_cast<const float4*>(Gs + s1 * L4);
            const float4* k1p = reinterpret_cast<const float4*>(Ks + s1 * L4);
            const float4* g2p = reinterpret_cast<const float4*>(Gs + s2 * L4);
            const float4* k2p = reinterpret_cast<const float4*>(Ks + s2 * L4);
            float pa1 = 0.f, pp1 = 0.f, pa2 = 0.f, pp2 = 0.f;
#pragma unroll 2
            for (int c = 0; c < DK / 4; ++c) {
                const float4 g = gt[c], q = qt[c], ga = g1p[c], ka = k1p[c], gb = g2p[c], kb = k2p[c];
                const float a0 = __builtin_amdgcn_exp2f(g.x - ga.x) * ka.x;
                const float a1 = __builtin_amdgcn_exp2f(g.y - ga.y) * ka.y;
                const float a2 = __builtin_amdgcn_exp2f(g.z - ga.z) * ka.z;
                const float a3 = __builtin_amdgcn_exp2f(g.w - ga.w) * ka.w;
                const float b0 = __builtin_amdgcn_exp2f(g.x - gb.x) * kb.x;
                const float b1 = __builtin_amdgcn_exp2f(g.y - gb.y) * kb.y;
                const float b2 = __builtin_amdgcn_exp2f(g.z - gb.z) * kb.z;
                const float b3 = __builtin_amdgcn_exp2f(g.w - gb.w) * kb.w;
                pp1 += q.x * a0 + q.y * a1 + q.z * a2 + q.w * a3;
                pp2 += q.x * b0 + q.y * b1 + q.z * b2 + q.w * b3;
                if constexpr (GDN) {
                    const float4 k = kt[c];
                    pa1 += k.x * a0 + k.y * a1 + k.z * a2 + k.w * a3;
                    pa2 += k.x * b0 + k.y * b1 + k.z * b2 + k.w * b3;
                }
            }
            if constexpr (GDN) Am[t * kC + s1] = bet[t] * pa1;
            Pm[t * kLT + s1] = pp1;
            if (s2 < t) {
                if constexpr (GDN) Am[t * kC + s2] = bet[t] * pa2;
                Pm[t * kLT + s2] = pp2;
            }
        }
        if (tid < 4 * kC) {  // diagonal of P: q_t . k_t, four lanes per token
            const int t = tid >> 2, part = tid & 3;
            const float4* qa = reinterpret_cast<const float4*>(Qs + t * L4) + part * (DK / 16);
            const float4* ka = reinterpret_cast<const float4*>(Ks + t * L4) + part * (DK / 16);
            float pp = 0.f;
#pragma unroll
            for (int c = 0; c < DK / 16; ++c) {
                const float4 a = qa[c], b = ka[c];
                pp += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
            }
            pp += dpp_move<0xB1>(pp);  // lane ^ 1
            pp += dpp_move<0x4E>(pp);  // lane ^ 2
            if (part == 0) Pm[t * kLT + t] = pp;
        }
        for (int x = tid; x < kC * DK; x += kThreads) {
            const int t = x / DK, c = x - t * DK, y = t * L4 + c, z = t * L1 + c;
            const float g = Gs[y];
            const float gam = __builtin_amdgcn_exp2f(g);
            Qg[z] = Qs[y] * gam;
            Kt[z] = Ks[y] * __builtin_amdgcn_exp2f(Gs[(kC - 1) * L4 + c] - g);
            if constexpr (GDN) Rw[z] = -(bet[t] * Ks[y] * gam);
        }
        __syncthreads();
        // c += A B^T over `steps` key steps from k0, A and B both read along key rows
        // (A: 32 token rows, B: 32 state rows, row stride L1)
        auto rows_dot = [&](const float* A, const float* B, auto steps, int k0, f32x16 c) {
            return chain<decltype(steps)::value>([&](int s) { return A[l32 * L1 + 2 * (k0 + s) + kg]; },
                                                 [&](int s) { return B[l32 * L1 + 2 * (k0 + s) + kg]; }, c);
        };
        using Full = std::integral_constant<int, DK / 2>;
        using Half = std::integral_constant<int, DK / 4>;
        // c += P U or T X on value columns 32 I ..: B read along token rows of Us
        auto tok_dot = [&](const float* A, int I, f32x16 c) {
            return chain<kC / 2>([&](int s) { return A[l32 * kLT + 2 * s + kg]; },
                                 [&](int s) { return Us[(2 * s + kg) * kSL + 32 * I + l32]; }, c);
        };
        auto store_o = [&](int I, const f32x16& c) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                if (c0 + t < T) io<E>::store(o, v_base + (size_t)(c0 + t) * dv + r0 + 32 * I + l32, c[e]);
            }
        };
        if constexpr (GDN) {
            // U = T (R_v - R_w S^T) = T X.  Phase A: wave 0 inverts I + A while
            // waves 1 and 2 form X in place of R_v (value columns 32 (w - 1) ..)
            // and wave 3 starts O = (Q gamma) S^T on value columns 0 .. 31.
            f32x16 oacc = {};
            if (w == 0) {
                const float4* A4 = reinterpret_cast<const float4*>(Am);
                float xcol[kC];
                // row r + 1 of A is in flight while row r is reduced
                float4 cur[kC / 4], nxt[kC / 4];
                cur[0] = A4[kC / 4];
                xcol[0] = l32 == 0 ? 1.f : 0.f;
#pragma unroll
                for (int r = 1; r < kC; ++r) {
                    if (r + 1 < kC) {
                        // the offset is tied to the previous row's result, so
                        // these loads issue after it and one row ahead of use
                        int off = (r + 1) * (kC / 4);
                        asm volatile("" : "+v"(off) : "v"(xcol[r - 1]));
#pragma unroll
                        for (int m = 0; m < (r + 4) / 4; ++m) nxt[m] = A4[off + m];
                    }
                    float acc = r == l32 ? 1.f : 0.f;
#pragma unroll
                    for (int j = 0; j < r; ++j) {
                        const float4 aj = cur[j / 4];
                        const float av = (j & 3) == 0 ? aj.x : (j & 3) == 1 ? aj.y : (j & 3) == 2 ? aj.z : aj.w;
                        acc -= av * xcol[j];
                    }
                    xcol[r] = acc;
                    if (r + 1 < kC) {
#pragma unroll
                        for (int m = 0; m < (r + 4) / 4; ++m) cur[m] = nxt[m];
                    }
                }
                if (kg == 0) {
#pragma unroll
                    for (int r = 0; r < kC; ++r) Tm[r * kLT + l32] = xcol[r];
                }
            } else if (w < 3) {
                const int I = w - 1;
                f32x16 c;
#pragma unroll
                for (int e = 0; e < 16; ++e) c[e] = Us[row(e) * kSL + 32 * I + l32];
                c = rows_dot(Rw, Ss + 32 * I * L1, Full{}, 0, c);  // Rw holds -beta k gamma
#pragma unroll
                for (int e = 0; e < 16; ++e) Us[row(e) * kSL + 32 * I + l32] = c[e];
            } else {
                oacc = rows_dot(Qg, Ss, Full{}, 0, oacc);
            }
            __syncthreads();
            // Phase B: U = T X (waves 1, 2); waves 0 and 3 share (Q gamma) S^T on
            // value columns 32 .. 63, one half of the keys each.
            if (w == 1 || w == 2) {
                const int I = w - 1;
                const f32x16 c = tok_dot(Tm, I, f32x16{});
#pragma unroll
                for (int e = 0; e < 16; ++e) Us[row(e) * kSL + 32 * I + l32] = c[e];
            } else if (w == 0) {
                oacc = rows_dot(Qg, Ss + 32 * L1, Half{}, 0, oacc);
            } else {
                const f32x16 part = rows_dot(Qg, Ss + 32 * L1, Half{}, DK / 4, f32x16{});
#pragma unroll
                for (int e = 0; e < 16; ++e) Ob[e * 64 + lane] = part[e];
            }
            __syncthreads();
            // Phase C: O += P U (wave 3: columns 0 .. 31, wave 0: 32 .. 63) beside
            // the state update (no wave reads the old state any more).
            if (w == 3) {
                store_o(0, tok_dot(Pm, 0, oacc));
            } else if (w == 0) {
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[e] += Ob[e * 64 + lane];
                store_o(1, tok_dot(Pm, 1, oacc));
            }
        } else {
            // O = (Q gamma) S^T + P V: waves 2, 3 (value columns 32 (w - 2) ..)
            if (w >= 2) store_o(w - 2, tok_dot(Pm, w - 2, rows_dot(Qg, Ss + 32 * (w - 2) * L1, Full{}, 0, f32x16{})));
            __syncthreads();  // every read of the old state done
        }
        // S <- S diag(gamma_C) + U^T K~: 2 x NJ tiles; with the delta rule waves
        // 1 and 2 take most of them (0 and 3 are busy with O)
        for (int tl = 0; tl < 2 * NJ; ++tl) {
            const int owner = GDN ? (tl < 2 * NJ - 2 ? 1 + (tl & 1) : (tl == 2 * NJ - 2 ? 0 : 3)) : (tl & 3);
            if (owner != w) continue;
            const int I = tl / NJ, J = tl - I * NJ;
            const float gC = __builtin_amdgcn_exp2f(Gs[(kC - 1) * L4 + 32 * J + l32]);
            f32x16 c;
#pragma unroll
            for (int e = 0; e < 16; ++e) c[e] = Ss[(32 * I + row(e)) * L1 + 32 * J + l32] * gC;
            c = chain<kC / 2>([&](int s) { return Us[(2 * s + kg) * kSL + 32 * I + l32]; },
                              [&](int s) { return Kt[(2 * s + kg) * L1 + 32 * J + l32]; }, c);
#pragma unroll
            for (int e = 0; e < 16; ++e) Ss[(32 * I + row(e)) * L1 + 32 * J + l32] = c[e];
        }
    }
    __syncthreads();
    if (ST)
        for (int x = tid; x < kSL * DK; x += kThreads) ST[s_base + x] = Ss[x / DK * L1 + x % DK];
}

template <int MODE, int DK, typename E>
hipError_t launch_dk(int BH, int T, int dv, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* S0, void* o, float* ST,
                     hipStream_t s) {
    const E* qq = static_cast<const E*>(q);
    const E* kk = static_cast<const E*>(k);
    const E* vv = static_cast<const E*>(v);
    E* oo = static_cast<E*>(o);
    if constexpr (DK >= 32) {
        if (dv % kSL == 0) {
            hipLaunchKernelGGL((chunk_diag_mfma_kernel<MODE, DK, E>), dim3((unsigned)((size_t)BH * (dv / kSL))),
                               dim3(kThreads), 0, s, T, dv, qq, kk, vv, alpha, beta, S0, oo, ST);
            return hipGetLastError();
        }
    }
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
