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

// The same chunk algorithm with its products on the MFMA (float32, or split
// bf16 with bf16 data) for slices of 64 value rows and dk >= 32, on 8 waves.
// Per chunk:
//   1. q, k and log2 a arrive in registers, one key channel and a run of
//      consecutive tokens per thread; log2 a is summed along the chunk there,
//      the runs exchanging their totals through LDS.  The value slice goes to
//      LDS;
//   2. the operands of the decayed Gram are written from the registers:
//      splitting each pair's factor through the middle token m,
//      e^{g_t - g_s} = e^{g_t - g_m} e^{g_m - g_s}, turns A and P into two
//      plain 32x32 products of rows scaled by e^{+-(g - g_m)}.  In float32 that
//      is safe while every |g_t - g_m| stays within kSpread (log2 units); a
//      chunk with a wider span stores q, k and g instead and takes the
//      pairwise form (one exp2 per token pair and channel), with the scaled
//      copies q gamma, -k gamma and k e^{g_C - g}.  In a factored chunk
//      e^{g_m} moves onto the state's columns instead (S~ = S diag(e^{g_m})),
//      so that (Q gamma) S^T and (K gamma) S^T read the Gram's operands;
//   3. one phase: A and at once T = (I + diag(beta) A)^-1 on one wave, P on
//      another, X = V - (K gamma) S^T and O = (Q gamma) S^T on two each;
//   4. U = T diag(beta) X;
//   5. O += P U beside the state update S <- S diag(gamma_C) + U^T (K e^{g_C - g}),
//      all as 32x32 tiles (a factored chunk forms
//      (S~ + U^T (K e^{g_m - g})) diag(e^{g_C - g_m}) instead).
// With bf16 data the operands are stored as bf16 hi / lo planes by the code
// that forms them (the products' split done once), the token-long ones (U, P,
// the update's keys) transposed so that they are read as 16-byte rows.
// U = T (R_v - R_w S^T) = T diag(beta) (V - (K gamma) S^T) is the product
// T R_v - (T R_w) S^T grouped so that the key-long part does not wait for the
// inverse, with the strengths applied to the columns of T.
// T = (I + diag(bet) B)^-1 for the strictly lower part of the 32x32 matrix B,
// given as its transpose Bt (Bt[s][t] = B[t][s], row stride LB, 16-byte rows),
// into Tm (row stride LT): the two 16x16 diagonal blocks side by side on the two
// halves of the wave (lane (b, c) owns column c of block b) by right-looking
// substitution, x_i = [i == c] - bet_i acc_i, then acc_r += B_ri x_i for r > i
// (row i of Bt read as float4 rows ahead: each step waits on one product, not
// on a sum over every earlier row), then T10 = -D1 diag(bet) B10 D0 on the
// 16x16x4 fp32 MFMA.  The upper right block of Tm is not written: it stays zero
// from the start.  All 64 lanes of the wave take part.
template <int LB, int LT>
__device__ __forceinline__ void solve_unit_lower_t(const float* Bt, const float* bet, float* Tm, int lane) {
    const int b = (lane >> 4) & 1, c = lane & 15, kg = lane >> 5;
    const float* Bb = Bt + 16 * b * LB + 16 * b;  // Bb[i * LB + r] = B[16 b + r][16 b + i]
    float br[16], acc[16], x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        br[r] = bet[16 * b + r];
        acc[r] = 0.f;
    }
    constexpr int AH = 2;  // rows read ahead of their step (LDS latency, not the
                           // products, sets the pace of the substitution)
    f32x4 rw[AH + 1][4];   // 4-entry groups from (i + 1) / 4 on of rows i .. i + AH
    auto load_row = [&](int i, f32x4 (&dst)[4]) {
#pragma unroll
        for (int q = (i + 1) / 4; q < 4; ++q) dst[q] = *reinterpret_cast<const f32x4*>(&Bb[i * LB + 4 * q]);
    };
#pragma unroll
    for (int i = 0; i < AH; ++i) load_row(i, rw[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i + AH < 16) load_row(i + AH, rw[(i + AH) % (AH + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        const float xi = (i == c ? 1.f : 0.f) - br[i] * acc[i];
        x[i] = xi;
#pragma unroll
        for (int r = i + 1; r < 16; ++r) acc[r] = fmaf(rw[i % (AH + 1)][r >> 2][r & 3], xi, acc[r]);
    }
    if (kg == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(16 * b + r) * LT + 16 * b + c] = x[r];
    }
    // T10 = -D1 (diag(bet) B10) D0: lane (n16, g4) supplies contraction indices
    // 4 g4 .. 4 g4 + 3 and holds rows 4 g4 .. 4 g4 + 3 of column n16
    const int n16 = lane & 15, g4 = lane >> 4;
    f32x4 y = {}, t10 = {};
    const float bs = bet[16 + n16];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)  // B10[n16][4 g4 + kk] = Bt[4 g4 + kk][16 + n16]
        y = mfma4(Bt[(4 * g4 + kk) * LB + 16 + n16] * bs, Tm[(4 * g4 + kk) * LT + n16], y);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t10 = mfma4(Tm[(16 + n16) * LT + 16 + 4 * g4 + kk], y[kk], t10);
#pragma unroll
    for (int r = 0; r < 4; ++r) Tm[(16 + 4 * g4 + r) * LT + n16] = -t10[r];
}

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
    // With bf16 data, Qg, Rw and (in a factored chunk) QA, KA, KB hold bf16 hi / lo
    // planes instead of floats, split once by their producer rather than by every
    // product that reads them: row t of such an array is the hi parts of its d_k
    // keys, then the lo parts, in the row's L4 floats (LP bf16; 16-byte reads of
    // 16 rows stay conflict-free).  Kt holds the state update's keys as floats in
    // every chunk.
    constexpr bool PL = SPLIT;
    constexpr int LP = 2 * L4;
    // The operands of P U and of the state update, which run along tokens, are
    // held transposed in the same way (bf16 data): U^T [value][token] and the
    // update's keys Kt^T [key][token], row r the hi parts of its 32 tokens, then
    // the lo parts (LT2 bf16 per row: 16-byte reads of 16 rows conflict-free).
    constexpr int LT2 = 2 * kC + 8;
    // Gram operands: q e^{g - g_m}, k e^{g - g_m} and k e^{g_m - g} in a
    // factored chunk; q, k and the cumulative log2 decay g in a wide one
    __shared__ __align__(16) float QA[kC * L4];
    __shared__ __align__(16) float KA[kC * L4];
    __shared__ __align__(16) float KB[kC * L4];
    __shared__ __align__(16) float Qg[kC * L4];            // q * gamma
    // the state update's keys: k e^{g_m - g} (factored) or k e^{g_C - g} (wide)
    __shared__ __align__(16) float Kt[PL ? DK * LT2 / 2 : kC * L4];
    __shared__ __align__(16) float Rw[GDN ? kC * L4 : 4];  // -(k * gamma)
    __shared__ __align__(16) float Us[kC * LU];            // v slice, then X (without beta), then U
    // U^T planes: in Qg (free once the read-out's first product is done) with the
    // delta rule; gated linear attention (U = V) keeps V^T in an array of its own
    __shared__ __align__(16) float UTs[!GDN && PL ? kSL * LT2 / 2 : 4];
    __shared__ __align__(16) float Am[GDN ? kC * kLT : 1];  // A^T without beta (A strictly lower)
    __shared__ __align__(16) float Tm[GDN ? kC * kLT : 4];  // T
    __shared__ __align__(16) float Pm[kC * kLT];            // P (lower, inclusive; zero above; planes like U^T)
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
    // Per-head buffer resources: one instruction per load, its offset a 32-bit
    // register plus a constant, and reads past the sequence's end return zeros
    // (those tokens are masked where they are used).  Byte offsets stay below
    // 2^31 (checked at launch).
    auto rsrc = [](const void* base, size_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + qk_base, (size_t)T * DK * sizeof(E));
    const __amdgpu_buffer_rsrc_t rk = rsrc(k + qk_base, (size_t)T * DK * sizeof(E));
    const __amdgpu_buffer_rsrc_t ra = rsrc(alpha + qk_base, (size_t)T * DK * 4);
    const __amdgpu_buffer_rsrc_t rv = rsrc(v + v_base + r0, ((size_t)T * dv - r0) * sizeof(E));
    const __amdgpu_buffer_rsrc_t rb = rsrc(beta ? beta + (size_t)bh * T : alpha, beta ? (size_t)T * 4 : 0);
    auto ld_e = [](__amdgpu_buffer_rsrc_t r, int off) {
        if constexpr (std::is_same<E, uint16_t>::value)
            return (E)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        else
            return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    };
    auto ld_f = [](__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    };
    auto fetch = [&](int cn) {
        const int e0 = (cn + run * NQ) * DK + ch;  // element of (first token, channel) in the head
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            pq[m] = ld_e(rq, (e0 + m * DK) * (int)sizeof(E));
            pk[m] = ld_e(rk, (e0 + m * DK) * (int)sizeof(E));
            pa[m] = ld_f(ra, (e0 + m * DK) * 4);
        }
        const int v0 = (cn + tid / kSL) * dv + tid % kSL;
#pragma unroll
        for (int m = 0; m < NV; ++m) pv[m] = ld_e(rv, (v0 + m * (kThreadsM / kSL) * dv) * (int)sizeof(E));
        if (GDN && tid < kC) pb = ld_f(rb, (cn + tid) * 4);
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
            const float vx = x / kSL < o0 ? to_f32(pv[m]) : 0.f;
            if constexpr (!GDN && PL) {  // U = V: V^T planes, (value, token) at value LT2 + token
                uint16_t* P = reinterpret_cast<uint16_t*>(UTs) + (x % kSL) * LT2 + x / kSL;
                P[0] = f32_to_bf16(vx);  // exact: bf16 data
                P[kC] = 0;
            } else {
                Us[x / kSL * LU + x % kSL] = vx;
            }
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
        int b4 = run * NQ * L4 + ch, p4 = 2 * run * NQ * L4 + ch;
        asm volatile("" : "+v"(b4), "+v"(p4));
        // element (t, ch) of an operand array: a float at t L4 + ch, or hi / lo bf16
        // at t LP + ch and t LP + DK + ch
        auto put_op = [&](float* X, int m, float x) {
            if constexpr (PL) {
                uint16_t* P = reinterpret_cast<uint16_t*>(X) + p4 + m * LP;
                const uint16_t h = f32_to_bf16(x);
                P[0] = h;
                P[DK] = f32_to_bf16(x - bf16_to_f32(h));
            } else {
                X[b4 + m * L4] = x;
            }
        };
        auto put = [&](auto factored) {
            constexpr bool F = decltype(factored)::value;
            // factored: gamma_t = e^{g_t - g_m} e^{g_m}, with e^{g_m} moved onto the
            // state's columns (below), so that (Q gamma) S^T = QA (S e^{g_m})^T and
            // (K gamma) S^T = KA (S e^{g_m})^T need no copies of their own; k e^{g_C - g}
            // is not formed either (the state update scales by e^{g_C - g_m} per column)
            if (run == 0) {
                sIn[ch] = F ? 1.f : __builtin_amdgcn_exp2f(gc);
                sOut[ch] = F ? __builtin_amdgcn_exp2f(gc - gm) : 1.f;
            }
            float kt[NQ];  // the state update's keys of this thread's tokens
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const bool in = run * NQ + m < o0;
                const float qq = in ? to_f32(pq[m]) : 0.f, kk = in ? to_f32(pk[m]) : 0.f;
                const int y = b4 + m * L4;
                if constexpr (F) {
                    const float up = __builtin_amdgcn_exp2f(g[m] - gm), dn = __builtin_amdgcn_exp2f(gm - g[m]);
                    const float qu = qq * up, ku = kk * up, kd = kk * dn;
                    put_op(QA, m, qu);
                    if constexpr (GDN) put_op(KA, m, ku);
                    put_op(KB, m, kd);
                    kt[m] = kd;
                } else {
                    const float gam = __builtin_amdgcn_exp2f(g[m]);
                    put_op(Qg, m, qq * gam);
                    kt[m] = kk * __builtin_amdgcn_exp2f(gc - g[m]);
                    if constexpr (GDN) put_op(Rw, m, -(kk * gam));
                    QA[y] = qq;
                    KA[y] = kk;
                    KB[y] = g[m];
                }
            }
            if constexpr (PL) {
                // Kt^T planes: this thread's NQ consecutive tokens of key ch, one vector
                // store per plane
                typedef __bf16 bfq __attribute__((ext_vector_type(NQ)));
                bfq hi, lo;
#pragma unroll
                for (int m = 0; m < NQ; ++m) {
                    hi[m] = static_cast<__bf16>(kt[m]);
                    lo[m] = static_cast<__bf16>(kt[m] - static_cast<float>(hi[m]));
                }
                uint16_t* P = reinterpret_cast<uint16_t*>(Kt) + ch * LT2 + run * NQ;
                *reinterpret_cast<bfq*>(P) = hi;
                *reinterpret_cast<bfq*>(P + kC) = lo;
            } else {
#pragma unroll
                for (int m = 0; m < NQ; ++m) Kt[b4 + m * L4] = kt[m];
            }
        };
        if (wide) {
            put(std::false_type{});
        } else {
            put(std::true_type{});
            // S <- S diag(e^{g_m}) in place, tile w on wave w (the state update starts from
            // it); e^{g_m} of key column c from the run totals: the runs before the middle
            if (w < 2 * NJ) {
                const int I = w / NJ, J = w - I * NJ, col = 32 * J + l32;
                float gmc = 0.f;
#pragma unroll
                for (int r = 0; r < kC / 2 / NQ; ++r) gmc += Gr[r * DK + col];
                const float f = __builtin_amdgcn_exp2f(gmc);
#pragma unroll
                for (int e = 0; e < 16; ++e) Ss[(32 * I + row(e)) * L4 + col] *= f;
            }
        }
        if (n + 1 < nchunks) fetch(c0 + kC);
        __syncthreads();
        // P[t][s]: a float, or (bf16 data) hi / lo at t LT2 + s and t LT2 + kC + s
        auto put_pm = [&](int t, int si, float x) {
            if constexpr (PL) {
                uint16_t* P = reinterpret_cast<uint16_t*>(Pm) + t * LT2 + si;
                const uint16_t h = f32_to_bf16(x);
                P[0] = h;
                P[kC] = f32_to_bf16(x - bf16_to_f32(h));
            } else {
                Pm[t * kLT + si] = x;
            }
        };
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
                if constexpr (GDN) Am[s1 * kLT + t] = pa1;
                put_pm(t, s1, pp1);
                if (s2 < t) {
                    if constexpr (GDN) Am[s2 * kLT + t] = pa2;
                    put_pm(t, s2, pp2);
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
                if (part == 0) put_pm(td, td, pp);
            }
            __syncthreads();
        }
        // c += A B^T over G groups of 16 keys from key 16 g0, A in planes and B in
        // planes (dot_pp) or floats (dot_pf, split here): three bf16 MFMAs per group,
        // hi hi + hi lo + lo hi; each group's operands are read one group ahead
        auto plane8 = [&](const float* X, int g) {
            return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(X) + l32 * LP + 16 * g + 8 * kg);
        };
        auto plane8lo = [&](const float* X, int g) {
            return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(X) + l32 * LP + DK + 16 * g + 8 * kg);
        };
        auto dot_pp = [&](const float* A, const float* B, auto groups, int g0, f32x16 c) {
            constexpr int G = decltype(groups)::value;
            bf16x8 ah = plane8(A, g0), al = plane8lo(A, g0), bh = plane8(B, g0), bl = plane8lo(B, g0);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                bf16x8 ahn = ah, aln = al, bhn = bh, bln = bl;
                if (i + 1 < G) {
                    ahn = plane8(A, g0 + i + 1);
                    aln = plane8lo(A, g0 + i + 1);
                    bhn = plane8(B, g0 + i + 1);
                    bln = plane8lo(B, g0 + i + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                ah = ahn;
                al = aln;
                bh = bhn;
                bl = bln;
            }
            return c;
        };
        auto dot_pf = [&](const float* A, const float* B, auto groups, int g0, f32x16 c) {
            constexpr int G = decltype(groups)::value;
            const float* bp = B + l32 * L4 + 16 * g0 + 8 * kg;
            bf16x8 ah = plane8(A, g0), al = plane8lo(A, g0);
            f32x8 b = lds_f32x8(bp);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                bf16x8 ahn = ah, aln = al;
                f32x8 bn = b;
                if (i + 1 < G) {
                    ahn = plane8(A, g0 + i + 1);
                    aln = plane8lo(A, g0 + i + 1);
                    bn = lds_f32x8(bp + 16 * (i + 1));
                }
                bf16x8 bh, bl;
                split_bf16(b, bh, bl);
                __builtin_amdgcn_sched_barrier(0);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                ah = ahn;
                al = aln;
                b = bn;
            }
            return c;
        };
        // c += X Y^T over keys [2 k0, 2 k0 + 2 STEPS) with X an operand array (planes
        // with bf16 data) and Y the state (floats)
        auto op_dot_s = [&](const float* X, const float* Y, auto steps, int k0, f32x16 c) {
            constexpr int STEPS = decltype(steps)::value;
            if constexpr (PL)
                return dot_pf(X, Y, std::integral_constant<int, STEPS / 8>{}, k0 / 8, c);
            else
                return rows_dot(X, Y, steps, k0, c);
        };
        // factored Gram tile: C[t][s] = sum_i X_ti e^{g_ti - g_mi} k_si e^{g_mi - g_si}
        auto gram = [&](const float* X) {
            if constexpr (PL)
                return dot_pp(X, KB, std::integral_constant<int, DK / 16>{}, 0, f32x16{});
            else
                return rows_dot(X, KB, Full{}, 0, f32x16{});
        };
        // the factored P (lower, inclusive) into Pm.  With bf16 data it is formed
        // transposed, C[s][t] = P[t][s], so that a lane holds row t = l32 of P with
        // four consecutive s per element group: 8-byte plane stores.
        auto store_p = [&]() {
            if constexpr (PL) {
                const f32x16 c = dot_pp(KB, QA, std::integral_constant<int, DK / 16>{}, 0, f32x16{});
                uint16_t* P = reinterpret_cast<uint16_t*>(Pm) + l32 * LT2 + 4 * kg;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    bf16x4 hi, lo;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = 8 * b + 4 * kg + r <= l32 ? c[4 * b + r] : 0.f;
                        hi[r] = static_cast<__bf16>(x);
                        lo[r] = static_cast<__bf16>(x - static_cast<float>(hi[r]));
                    }
                    *reinterpret_cast<bf16x4*>(P + 8 * b) = hi;
                    *reinterpret_cast<bf16x4*>(P + kC + 8 * b) = lo;
                }
            } else {
                const f32x16 c = gram(QA);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = row(e);
                    Pm[t * kLT + l32] = l32 <= t ? c[e] : 0.f;
                }
            }
        };
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
            const f32x16 c = op_dot_s(wide ? Qg : QA, Ss + 32 * I * L4, std::integral_constant<int, DK / 8>{}, 3 * DK / 8,
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
        const float* KS = Kt;
        auto s_init = [&](int tl) {
            const int I = tl / NJ, J = tl - I * NJ;
            const float f = sIn[32 * J + l32];
            f32x16 c;
#pragma unroll
            for (int e = 0; e < 16; ++e) c[e] = Ss[(32 * I + row(e)) * L4 + 32 * J + l32] * f;
            return c;
        };
        float* UT = GDN ? Qg : UTs;
        // hi / lo parts of tokens 16 i + 8 kg .. + 7 of row r of a transposed plane array
        auto tplane = [&](const float* X, int r, int i, int part) {
            return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(X) + r * LT2 + part * kC +
                                                    16 * i + 8 * kg);
        };
        auto s_done = [&](int tl, f32x16 c) {
            const int I = tl / NJ, J = tl - I * NJ;
            if constexpr (PL) {
                const int ru = 32 * I + l32, rk = 32 * J + l32;
#pragma unroll
                for (int i = 0; i < kC / 16; ++i) {
                    const bf16x8 ah = tplane(UT, ru, i, 0), al = tplane(UT, ru, i, 1);
                    const bf16x8 bh = tplane(Kt, rk, i, 0), bl = tplane(Kt, rk, i, 1);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
                }
            } else {
                c = chain8_t<SPLIT, kC / 16>(
                    [&](int i) { return lds_col8<LU>(&Us[(16 * i + 8 * kg) * LU + 32 * I + l32]); },
                    [&](int i) { return lds_col8<L4>(&KS[(16 * i + 8 * kg) * L4 + 32 * J + l32]); }, c);
            }
            const float f = sOut[32 * J + l32];
#pragma unroll
            for (int e = 0; e < 16; ++e) Ss[(32 * I + row(e)) * L4 + 32 * J + l32] = c[e] * f;
        };
        // c += P U on value columns 32 I ..
        auto pu_dot = [&](int I, f32x16 c) {
            if constexpr (PL) {
                const int ru = 32 * I + l32;
#pragma unroll
                for (int i = 0; i < kC / 16; ++i) {
                    const bf16x8 ah = tplane(Pm, l32, i, 0), al = tplane(Pm, l32, i, 1);
                    const bf16x8 bh = tplane(UT, ru, i, 0), bl = tplane(UT, ru, i, 1);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
                }
                return c;
            } else {
                return tok_dot(Pm, I, c);
            }
        };
        f32x16 oacc = {};
        if constexpr (GDN) {
            // 3. One phase: wave 0 forms A and at once inverts I + diag(beta) A with the
            // blocked solve (its own writes of A need only its LDS counter); wave 1 forms P,
            // waves 2, 3 diag(beta) X, X = V - (K gamma) S^T, in place of V on value columns
            // 32 (w - 2) .., and waves 6, 7 O = (Q gamma) S^T on value tiles 0, 1.  None of
            // them reads another's result.
            if (w == 0) {
                if (!wide) {
                    // c[e] = A[t][s] for t = row(e), s = l32: row s of A^T, tokens
                    // 8 b + 4 kg .. + 3 in elements 4 b .. 4 b + 3 (16-byte stores)
                    const f32x16 c = gram(KA);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        f32x4 a;
#pragma unroll
                        for (int r = 0; r < 4; ++r) a[r] = 8 * b + 4 * kg + r > l32 ? c[4 * b + r] : 0.f;
                        *reinterpret_cast<f32x4*>(&Am[l32 * kLT + 8 * b + 4 * kg]) = a;
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
                solve_unit_lower_t<kLT, kLT>(Am, bet, Tm, lane);
            } else if (w == 1) {
                if (!wide) store_p();
            } else if (w < 4) {
                const int I = w - 2;
                const float sg = wide ? 1.f : -1.f;
                f32x16 c;
#pragma unroll
                for (int e = 0; e < 16; ++e) c[e] = sg * Us[row(e) * LU + 32 * I + l32];
                // wide: V + Rw S^T (Rw holds -k gamma); factored: -(-V + KA (S e^{g_m})^T)
                c = op_dot_s(wide ? Rw : KA, Ss + 32 * I * L4, Full{}, 0, c);
#pragma unroll
                for (int e = 0; e < 16; ++e) Us[row(e) * LU + 32 * I + l32] = sg * bet[row(e)] * c[e];
            } else if (w >= 6) {
                oacc = op_dot_s(wide ? Qg : QA, Ss + 32 * (w - 6) * L4, Full{}, 0, oacc);
            }
            __syncthreads();
            // 4. U = T (diag(beta) X) (waves 1, 2; as U^T planes with bf16 data) while the
            // others read their first state tile; then O += P U (waves 6, 7) beside the
            // state update, state tiles i and i + 6 on wave i < 6.
            const bool has_tile = w < 6 && w < 2 * NJ;
            f32x16 sreg;
            if (w == 1 || w == 2) {
                const int I = w - 1;
                const f32x16 u = tok_dot(Tm, I, f32x16{});
                if constexpr (PL) {
                    // lane: value 32 I + l32, tokens 8 b + 4 kg .. + 3 in elements 4 b .. 4 b + 3
                    uint16_t* P = reinterpret_cast<uint16_t*>(UT) + (32 * I + l32) * LT2 + 4 * kg;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        bf16x4 hi, lo;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            hi[r] = static_cast<__bf16>(u[4 * b + r]);
                            lo[r] = static_cast<__bf16>(u[4 * b + r] - static_cast<float>(hi[r]));
                        }
                        *reinterpret_cast<bf16x4*>(P + 8 * b) = hi;
                        *reinterpret_cast<bf16x4*>(P + kC + 8 * b) = lo;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) Us[row(e) * LU + 32 * I + l32] = u[e];
                }
            } else if (has_tile) {
                sreg = s_init(w);
            }
            __syncthreads();
            if (w >= 6) store_o(w - 6, pu_dot(w - 6, oacc));
            if (has_tile) s_done(w, (w == 1 || w == 2) ? s_init(w) : sreg);
            if (w < 6 && w + 6 < 2 * NJ) s_done(w + 6, s_init(w + 6));
        } else {
            // P (wave 0) beside O = (Q gamma) S^T on value columns 32 (w - 2) ..
            // (waves 2, 3; waves 1, 5 the last key quarter of tiles 0, 1)
            if (w == 0) {
                if (!wide) store_p();
            } else if (w == 2 || w == 3) {
                oacc = op_dot_s(wide ? Qg : QA, Ss + 32 * (w - 2) * L4, OHead{}, 0, oacc);
            } else if (kSplitO && (w == 1 || w == 5)) {
                o_tail(w == 5);
            }
            __syncthreads();  // P done, every read of the old state done
            // O += P U (waves 2, 3) beside the state update: state tiles i and i + 6 go to
            // the wave in position i of 0, 1, 4, 5, 6, 7
            const int slot = w < 2 ? w : w - 2;
            if (w == 2 || w == 3) {
                store_o(w - 2, pu_dot(w - 2, o_add_tail(w - 2, oacc)));
            } else {
                if (slot < 2 * NJ) s_done(slot, s_init(slot));
                if (slot + 6 < 2 * NJ) s_done(slot + 6, s_init(slot + 6));
            }
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
        // the MFMA kernel's per-head byte offsets are 32-bit
        const bool fits = (size_t)T * (size_t)(dv > DK ? dv : DK) * 4 < (size_t(1) << 31);
        if (dv % kSL == 0 && fits) {
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
