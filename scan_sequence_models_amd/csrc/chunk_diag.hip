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
#include "solve.hpp"

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
    int bh, sl;
    unit_part(blockIdx.x, gridDim.x / slices, slices, bh, sl);  // a head's slices share its q, k reads in L2
    const int r0 = sl * SL;
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
//   1. q, k and log2 a arrive in registers, one key channel and a run of
//      consecutive tokens per thread; log2 a is summed along the chunk there,
//      the runs exchanging their totals through LDS.  The value slice goes to
//      LDS;
//   2. the scaled copies q gamma and -k gamma (and, in a wide chunk,
//      k e^{g_C - g}) are written from the registers, and so are the operands
//      of the decayed Gram:
//      splitting each pair's factor through the middle token m,
//      e^{g_t - g_s} = e^{g_t - g_m} e^{g_m - g_s}, turns A and P into two
//      plain 32x32 products of rows scaled by e^{+-(g - g_m)}.  In float32 that
//      is safe while every |g_t - g_m| stays within kSpread (log2 units); a
//      chunk with a wider span stores q, k and g instead and takes the
//      pairwise form (one exp2 per token pair and channel);
//   3. A and P on two waves beside X = V - (K gamma) S^T on the other two;
//   4. T = (I + diag(beta) A)^-1 by one wave (a lane per column, forward
//      substitution with the rows of A read as float4) beside
//      O = (Q gamma) S^T on the other three;
//   5. U = T diag(beta) X; then O += P U beside the state update
//      S <- S diag(gamma_C) + U^T (K e^{g_C - g}), all as 32x32 tiles (a
//      factored chunk scales by e^{g_C - g_m} per column instead of forming
//      K e^{g_C - g}).
// U = T (R_v - R_w S^T) = T diag(beta) (V - (K gamma) S^T) is the product
// T R_v - (T R_w) S^T grouped so that the key-long part does not wait for the
// inverse, with the strengths applied to the columns of T.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
constexpr int kSL = 64;      // value rows per workgroup
constexpr int kThreadsM = 512;  // 8 waves, two per SIMD
constexpr int kLT = kC + 4;  // row stride of the 32x32 T and P tiles (float4 rows)
// widest |g_t - g_m| (log2) of the factored Gram: its operands stay within
// 2^(+-64), far from float32 overflow, and a term lost to underflow there is
// below 2^-62 of the unit-scale ones
constexpr float kSpread = 64.f;

template <int MODE, int DK, typename E>
__global__ __launch_bounds__(kThreadsM) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunk_diag_mfma_kernel(
    int T, int dv, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    E* __restrict__ o, float* __restrict__ ST) {
    constexpr bool GDN = MODE == 0;
    constexpr int NJ = DK / 32;
    // bf16 data: the products in split bf16 (about 16 significant bits each)
    constexpr bool SPLIT = std::is_same<E, uint16_t>::value;              // 32-column tiles of a key-wide row
    constexpr int NQ = kC * DK / kThreadsM;   // tokens per thread, all of one key channel
    constexpr int NR = kThreadsM / DK;        // runs of NQ tokens per chunk
    constexpr int NV = kC * kSL / kThreadsM;  // value elements per thread and chunk
    static_assert((kC / 2) % NQ == 0, "the middle token m = kC/2 - 1 ends a run");
    static_assert(DK < 64 || kC * (DK + 4) >= 2048, "KA holds two partial O tiles");
    // Row strides: 16-byte rows.  The pairwise Gram reads float4 runs of
    // channels with one token per lane, and the MFMA operands along a row come
    // in 16-byte reads (eight k per lane half: k = 16 i + 8 kg + j), both
    // conflict-free with 16 lanes on rows 4 banks apart; down a column, the
    // rows r and r + 8 of the two lane halves land 32 banks apart.
    constexpr int L4 = DK + 4;
    constexpr int LU = kSL + 4;
    // Gram operands: q e^{g - g_m}, k e^{g - g_m} and k e^{g_m - g} in a
    // factored chunk; q, k and the cumulative log2 decay g in a wide one
    __shared__ __align__(16) float QA[kC * L4];
    __shared__ __align__(16) float KA[kC * L4];
    __shared__ __align__(16) float KB[kC * L4];
    __shared__ __align__(16) float Qg[kC * L4];            // q * gamma
    __shared__ __align__(16) float Kt[kC * L4];            // k * e^{g_C - g} (wide chunks)
    __shared__ __align__(16) float Rw[GDN ? kC * L4 : 4];  // -(k * gamma)
    __shared__ __align__(16) float Us[kC * LU];            // v slice, then X (without beta), then U
    __shared__ __align__(16) float Am[GDN ? kC * kC : 1];  // A without beta (strictly lower)
    __shared__ __align__(16) float Tm[GDN ? kC * kLT : 4];  // T
    __shared__ __align__(16) float Pm[kC * kLT];            // P (lower, inclusive; zero above)
    __shared__ __align__(16) float Ss[kSL * L4];            // state slice
    __shared__ float Gr[NR * DK];                // run totals of log2 a
    __shared__ float sIn[DK];                    // per-channel factors of the state update:
    __shared__ float sOut[DK];                   // e^{g_m}, e^{g_C - g_m} (wide: gamma_C, 1)
    __shared__ __align__(16) float bet[kC];
    __shared__ int wflag[kThreadsM / 64];        // a wave holds a chunk too wide to factor

    const int slices = dv / kSL;
    int bh, sl;
    unit_part(blockIdx.x, gridDim.x / slices, slices, bh, sl);  // a head's slices share its q, k reads in L2
    const int r0 = sl * kSL;
    int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int l32 = lane & 31, kg = lane >> 5;
    int ch = tid % DK, run = tid / DK;  // this thread's key channel and run of tokens
    const size_t qk_base = (size_t)bh * T * DK;
    const size_t v_base = (size_t)bh * T * dv;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;
    // accumulator element e of a 32x32 tile: row 8 (e / 4) + 4 kg + e % 4, column l32
    auto row = [&](int e) { return 8 * (e >> 2) + 4 * kg + (e & 3); };

    for (int x = tid; x < kSL * DK; x += kThreadsM) Ss[x / DK * L4 + x % DK] = S0 ? S0[s_base + x] : 0.f;
    for (int x = tid; x < kC * kLT; x += kThreadsM) Pm[x] = 0.f;
    if constexpr (GDN)
        for (int x = tid; x < kC * kLT; x += kThreadsM) Tm[x] = 0.f;  // T's upper right block stays zero

    // The next chunk's inputs are fetched into registers while this chunk
    // computes (every wave works on the chunk; nothing else hides HBM latency).
    // The loads are unconditional, from a token index clamped into the
    // sequence, and keep the raw element; masking and conversion happen when
    // they are used, so no load waits inside the fetch.
    E pq[NQ], pk[NQ], pv[NV];
    float pa[NQ], pb = 0.f;
    auto fetch = [&](int cn) {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int t = min(cn + run * NQ + m, T - 1);
            const size_t gi = qk_base + (size_t)t * DK + ch;
            pq[m] = q[gi];
            pk[m] = k[gi];
            pa[m] = alpha[gi];
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreadsM, t = min(cn + x / kSL, T - 1);
            pv[m] = v[v_base + (size_t)t * dv + r0 + x % kSL];
        }
        if (GDN && tid < kC) pb = beta[(size_t)bh * T + min(cn + tid, T - 1)];
    };
    fetch(0);

    // c += A B^T over `steps` key steps (two keys each) from step k0, A and B
    // both read along key rows (A: 32 token rows, B: 32 state rows)
    auto rows_dot = [&](const float* A, const float* B, auto steps, int k0, f32x16 c) {
        constexpr int G = decltype(steps)::value / 8;
        return chain8_t<SPLIT, G>([&](int i) { return lds_f32x8(&A[l32 * L4 + 2 * k0 + 16 * i + 8 * kg]); },
                                  [&](int i) { return lds_f32x8(&B[l32 * L4 + 2 * k0 + 16 * i + 8 * kg]); }, c);
    };
    using Full = std::integral_constant<int, DK / 2>;
    // c += P U or T X on value columns 32 I ..: B read along token rows of Us
    auto tok_dot = [&](const float* A, int I, f32x16 c) {
        return chain8_t<SPLIT, kC / 16>(
            [&](int i) { return lds_f32x8(&A[l32 * kLT + 16 * i + 8 * kg]); },
            [&](int i) { return lds_col8<LU>(&Us[(16 * i + 8 * kg) * LU + 32 * I + l32]); }, c);
    };

    const int nchunks = (T + kC - 1) / kC;
    for (int n = 0; n < nchunks; ++n) {
        // The lane indices are opaque to the compiler from here on, so the
        // address arithmetic built on them is redone in the loop rather than
        // hoisted out of it into live registers.
        asm volatile("" : "+v"(tid), "+v"(lane), "+v"(l32), "+v"(kg), "+v"(ch), "+v"(run));
        const int c0 = n * kC;
        const int o0 = min(kC, T - c0);  // tokens of this chunk inside the sequence
        __syncthreads();  // the previous chunk is done with every array
        // 1. past T: identity tokens (a = 1, beta = 0, q = k = v = 0)
        float g[NQ];
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            acc += run * NQ + m < o0 ? __log2f(pa[m]) : 0.f;
            g[m] = acc;
        }
        Gr[run * DK + ch] = acc;
        if (tid < kC) bet[tid] = tid < o0 ? pb : 0.f;
        __syncthreads();
        float off = 0.f, gm = 0.f, gc = 0.f;  // this run's offset, g_m, g_C
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float x = Gr[r * DK + ch];
            if (r < run) off += x;
            if (r < kC / 2 / NQ) gm += x;
            gc += x;
        }
        bool narrow = true;  // false for a zero, infinite or NaN gate too
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            g[m] += off;
            narrow = narrow && __builtin_fabsf(g[m] - gm) <= kSpread;
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreadsM;
            Us[x / kSL * LU + x % kSL] = x / kSL < o0 ? to_f32(pv[m]) : 0.f;
        }
        // one flag per wave, one barrier (the flags are next written after the
        // following chunk's first barrier)
        const bool wave_wide = __builtin_amdgcn_ballot_w64(!narrow) != 0;  // all lanes vote
        if (lane == 0) wflag[w] = wave_wide;
        __syncthreads();
        bool wide = false;
#pragma unroll
        for (int i = 0; i < kThreadsM / 64; ++i) wide |= wflag[i] != 0;
        // 2. scaled copies and Gram operands.  The bases are opaque to the
        // compiler, so each store below is one base register plus an immediate
        // offset instead of an address hoisted out of the chunk loop.
        int b4 = run * NQ * L4 + ch;
        asm volatile("" : "+v"(b4));
        auto put = [&](auto factored) {
            constexpr bool F = decltype(factored)::value;
            // factored: gamma_t = e^{g_t - g_m} e^{g_m}, and k e^{g_C - g} is not
            // formed (the state update scales by e^{g_C - g_m} per column instead)
            const float em = __builtin_amdgcn_exp2f(gm);
            if (run == 0) {
                sIn[ch] = F ? em : __builtin_amdgcn_exp2f(gc);
                sOut[ch] = F ? __builtin_amdgcn_exp2f(gc - gm) : 1.f;
            }
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const bool in = run * NQ + m < o0;
                const float qq = in ? to_f32(pq[m]) : 0.f, kk = in ? to_f32(pk[m]) : 0.f;
                const int y = b4 + m * L4;
                if constexpr (F) {
                    const float up = __builtin_amdgcn_exp2f(g[m] - gm), dn = __builtin_amdgcn_exp2f(gm - g[m]);
                    const float qu = qq * up, ku = kk * up;
                    QA[y] = qu;
                    Qg[y] = qu * em;
                    if constexpr (GDN) {
                        KA[y] = ku;
                        Rw[y] = -(ku * em);
                    }
                    KB[y] = kk * dn;
                } else {
                    const float gam = __builtin_amdgcn_exp2f(g[m]);
                    Qg[y] = qq * gam;
                    Kt[y] = kk * __builtin_amdgcn_exp2f(gc - g[m]);
                    if constexpr (GDN) Rw[y] = -(kk * gam);
                    QA[y] = qq;
                    KA[y] = kk;
                    KB[y] = g[m];
                }
            }
        };
        if (wide) put(std::false_type{});
        else put(std::true_type{});
        if (n + 1 < nchunks) fetch(c0 + kC);
        __syncthreads();
        if (wide) {
            // decayed Gram and scores over the strictly lower pairs s < t, two pairs (t, 2b)
            // and (t, 2b + 1) per thread so that they share the loads of token t: row t holds
            // ceil(t / 2) such blocks, floor(t^2 / 4) of them precede it, and rows 1 .. 31
            // hold exactly 256, one per thread of waves 0 .. 3 (the second pair of the last
            // block of an odd row is the diagonal, which is not stored here)
            static_assert(kC == 32 && kThreadsM >= 256, "one Gram block per thread");
            if (tid < 256) {
                const int p = tid;
                int t = (int)__builtin_sqrtf(4.f * (float)p + 1.f);
                if ((t * t) / 4 > p) --t;
                if (((t + 1) * (t + 1)) / 4 <= p) ++t;
                const int s1 = 2 * (p - (t * t) / 4), s2 = s1 + 1;
                const float4* gt = reinterpret_cast<const float4*>(KB + t * L4);
                const float4* kt = reinterpret_cast<const float4*>(KA + t * L4);
                const float4* qt = reinterpret_cast<const float4*>(QA + t * L4);
                const float4* g1p = reinterpret_cast<const float4*>(KB + s1 * L4);
                const float4* k1p = reinterpret_cast<const float4*>(KA + s1 * L4);
                const float4* g2p = reinterpret_cast<const float4*>(KB + s2 * L4);
                const float4* k2p = reinterpret_cast<const float4*>(KA + s2 * L4);
                float pa1 = 0.f, pp1 = 0.f, pa2 = 0.f, pp2 = 0.f;
#pragma unroll 2
                for (int c = 0; c < DK / 4; ++c) {
                    const float4 gg = gt[c], qv = qt[c], ga = g1p[c], ka = k1p[c], gb = g2p[c], kb = k2p[c];
                    const float a0 = __builtin_amdgcn_exp2f(gg.x - ga.x) * ka.x;
                    const float a1 = __builtin_amdgcn_exp2f(gg.y - ga.y) * ka.y;
                    const float a2 = __builtin_amdgcn_exp2f(gg.z - ga.z) * ka.z;
                    const float a3 = __builtin_amdgcn_exp2f(gg.w - ga.w) * ka.w;
                    const float b0 = __builtin_amdgcn_exp2f(gg.x - gb.x) * kb.x;
                    const float b1 = __builtin_amdgcn_exp2f(gg.y - gb.y) * kb.y;
                    const float b2 = __builtin_amdgcn_exp2f(gg.z - gb.z) * kb.z;
                    const float b3 = __builtin_amdgcn_exp2f(gg.w - gb.w) * kb.w;
                    pp1 += qv.x * a0 + qv.y * a1 + qv.z * a2 + qv.w * a3;
                    pp2 += qv.x * b0 + qv.y * b1 + qv.z * b2 + qv.w * b3;
                    if constexpr (GDN) {
                        const float4 kk = kt[c];
                        pa1 += kk.x * a0 + kk.y * a1 + kk.z * a2 + kk.w * a3;
                        pa2 += kk.x * b0 + kk.y * b1 + kk.z * b2 + kk.w * b3;
                    }
                }
                if constexpr (GDN) Am[t * kC + s1] = pa1;
                Pm[t * kLT + s1] = pp1;
                if (s2 < t) {
                    if constexpr (GDN) Am[t * kC + s2] = pa2;
                    Pm[t * kLT + s2] = pp2;
                }
            }
            if (tid >= 256 && tid < 256 + 4 * kC) {  // diagonal of P: q_t . k_t, four lanes per token
                const int td = (tid - 256) >> 2, part = tid & 3;
                const float4* qa = reinterpret_cast<const float4*>(QA + td * L4) + part * (DK / 16);
                const float4* ka = reinterpret_cast<const float4*>(KA + td * L4) + part * (DK / 16);
                float pp = 0.f;
#pragma unroll
                for (int c = 0; c < DK / 16; ++c) {
                    const float4 a = qa[c], b = ka[c];
                    pp += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
                }
                pp += dpp_move<0xB1>(pp);  // lane ^ 1
                pp += dpp_move<0x4E>(pp);  // lane ^ 2
                if (part == 0) Pm[td * kLT + td] = pp;
            }
            __syncthreads();
        }
        // factored Gram tile: C[t][s] = sum_i X_ti e^{g_ti - g_mi} k_si e^{g_mi - g_si}
        auto gram = [&](const float* X) { return rows_dot(X, KB, Full{}, 0, f32x16{}); };
        auto store_o = [&](int I, const f32x16& c) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                if (t < o0) io<E>::store(o, v_base + (size_t)(c0 + t) * dv + r0 + 32 * I + l32, c[e]);
            }
        };
        // O = (Q gamma) S^T: two waves on two SIMDs take the first three quarters of
        // the keys of one value tile each, and the two waves of a third SIMD the last
        // quarter of one tile each, their partial tiles passing through KA (free once
        // the Gram is done)
        constexpr bool kSplitO = DK >= 64;  // KA holds the two partial tiles
        using OHead = std::integral_constant<int, kSplitO ? 3 * DK / 8 : DK / 2>;
        auto o_tail = [&](int I) {
            const f32x16 c = rows_dot(Qg, Ss + 32 * I * L4, std::integral_constant<int, DK / 8>{}, 3 * DK / 8,
                                      f32x16{});
#pragma unroll
            for (int e = 0; e < 16; ++e) KA[I * 1024 + e * 64 + lane] = c[e];
        };
        auto o_add_tail = [&](int I, f32x16 c) {
            if constexpr (kSplitO) {
#pragma unroll
                for (int e = 0; e < 16; ++e) c[e] += KA[I * 1024 + e * 64 + lane];
            }
            return c;
        };
        // S <- S diag(gamma_C) + U^T (K e^{g_C - g}) as 2 NJ tiles of 32 x 32; a
        // factored chunk forms (S e^{g_m} + U^T (K e^{g_m - g})) e^{g_C - g_m}
        // column by column
        const float* KS = wide ? Kt : KB;
        auto s_init = [&](int tl) {
            const int I = tl / NJ, J = tl - I * NJ;
            const float f = sIn[32 * J + l32];
            f32x16 c;
#pragma unroll
            for (int e = 0; e < 16; ++e) c[e] = Ss[(32 * I + row(e)) * L4 + 32 * J + l32] * f;
            return c;
        };
        auto s_done = [&](int tl, f32x16 c) {
            const int I = tl / NJ, J = tl - I * NJ;
            c = chain8_t<SPLIT, kC / 16>(
                [&](int i) { return lds_col8<LU>(&Us[(16 * i + 8 * kg) * LU + 32 * I + l32]); },
                [&](int i) { return lds_col8<L4>(&KS[(16 * i + 8 * kg) * L4 + 32 * J + l32]); }, c);
            const float f = sOut[32 * J + l32];
#pragma unroll
            for (int e = 0; e < 16; ++e) Ss[(32 * I + row(e)) * L4 + 32 * J + l32] = c[e] * f;
        };
        f32x16 oacc = {};
        if constexpr (GDN) {
            // 3. A (wave 0) and P (wave 1) beside diag(beta) X, X = V - (K gamma) S^T,
            // in place of V on value columns 32 (w - 2) .. (waves 2, 3).  Waves 4 .. 7 wait:
            // splitting these products by key halves over the two waves of a SIMD, with
            // the partial tiles passed through LDS, was slower.
            if (w == 0) {
                if (!wide) {
                    const f32x16 c = gram(KA);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = row(e);
                        Am[t * kC + l32] = l32 < t ? c[e] : 0.f;
                    }
                }
            } else if (w == 1) {
                if (!wide) {
                    const f32x16 c = gram(QA);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = row(e);
                        Pm[t * kLT + l32] = l32 <= t ? c[e] : 0.f;
                    }
                }
            } else if (w < 4) {
                const int I = w - 2;
                f32x16 c;
#pragma unroll
                for (int e = 0; e < 16; ++e) c[e] = Us[row(e) * LU + 32 * I + l32];
                c = rows_dot(Rw, Ss + 32 * I * L4, Full{}, 0, c);  // Rw holds -k gamma
#pragma unroll
                for (int e = 0; e < 16; ++e) Us[row(e) * LU + 32 * I + l32] = bet[row(e)] * c[e];
            }
            __syncthreads();
            // 4. T = (I + diag(beta) A)^-1 (wave 0) beside O = (Q gamma) S^T on value columns
            // 32 (w - 1) .. (waves 1, 2; waves 3, 7 the last key quarter of tiles 0, 1)
            if (w == 0) {
                solve_unit_lower<kC, kLT>(Am, bet, Tm, lane);
            } else if (w < 3) {
                oacc = rows_dot(Qg, Ss + 32 * (w - 1) * L4, OHead{}, 0, oacc);
            } else if (kSplitO && (w == 3 || w == 7)) {
                o_tail(w == 7);
            }
            __syncthreads();
            // 5. U = T (diag(beta) X) (waves 1, 2) while the other waves read their state
            // tiles; then O += P U on the same value columns beside the state update.
            // State tile i goes to the wave in position i of 0, 3, 4, 5, 6, 7, 1, 2.
            const int slot = w == 0 ? 0 : w == 3 ? 1 : w >= 4 ? w - 2 : w + 5;
            const bool has_tile = slot < 2 * NJ;
            f32x16 sreg;
            if (w == 1 || w == 2) {
                const int I = w - 1;
                const f32x16 u = tok_dot(Tm, I, f32x16{});
#pragma unroll
                for (int e = 0; e < 16; ++e) Us[row(e) * LU + 32 * I + l32] = u[e];
            } else if (has_tile) {
                sreg = s_init(slot);
            }
            __syncthreads();
            if (w == 1 || w == 2) {
                store_o(w - 1, tok_dot(Pm, w - 1, o_add_tail(w - 1, oacc)));
                if (has_tile) s_done(slot, s_init(slot));
            } else if (has_tile) {
                s_done(slot, sreg);
            }
        } else {
            // P (wave 0) beside O = (Q gamma) S^T on value columns 32 (w - 2) ..
            // (waves 2, 3; waves 1, 5 the last key quarter of tiles 0, 1)
            if (w == 0) {
                if (!wide) {
                    const f32x16 c = gram(QA);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = row(e);
                        Pm[t * kLT + l32] = l32 <= t ? c[e] : 0.f;
                    }
                }
            } else if (w == 2 || w == 3) {
                oacc = rows_dot(Qg, Ss + 32 * (w - 2) * L4, OHead{}, 0, oacc);
            } else if (kSplitO && (w == 1 || w == 5)) {
                o_tail(w == 5);
            }
            __syncthreads();  // P done, every read of the old state done
            // state tile i goes to the wave in position i of 0, 1, 4, 5, 6, 7, 2, 3
            const int slot = w < 2 ? w : w >= 4 ? w - 2 : w + 4;
            if (w == 2 || w == 3) store_o(w - 2, tok_dot(Pm, w - 2, o_add_tail(w - 2, oacc)));
            if (slot < 2 * NJ) s_done(slot, s_init(slot));
        }
    }
    __syncthreads();
    if (ST)
        for (int x = tid; x < kSL * DK; x += kThreadsM) ST[s_base + x] = Ss[x / DK * L4 + x % DK];
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
                               dim3(kThreadsM), 0, s, T, dv, qq, kk, vv, alpha, beta, S0, oo, ST);
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
