// scan_bwd.hip -- gradient of the scan through the chunkwise form, float32.
//
// The forward is the chunkwise (UT) form of the gated delta rule (and of gated
// linear attention): with S the state entering a 32-token chunk, g the
// cumulative log decay inside it, gamma = e^g, Gamma_ts = e^{g_t - g_s}:
//
//   B = strict_lower(Gamma o K K^T),  A = diag(beta) B,  T = (I + A)^-1
//   X = diag(beta) V - diag(beta gamma) K S^T,   U = T X            (GLA: U = V)
//   P = lower(Gamma o Q K^T),   O = diag(gamma) Q S^T + P U
//   S' = gamma_C S + U^T diag(e^{g_C - g}) K
//
// (the prefix-scan notes, key design 2, give the affine state update; the
// chunk form is its unrolling over the chunk).  Its reverse mode, for incoming
// gradients dO and dS', is (Kd = diag(e^{g_C - g}) K, dX = T^T dU):
//
//   dS  = gamma_C dS' + dO^T diag(gamma) Q - dX^T diag(beta gamma) K
//   dU  = Kd dS'^T + P^T dO,     dP = lower(dO U^T)
//   dQ  = diag(gamma) dO S + (dP o Gamma) K
//   dK  = diag(e^{g_C-g}) U dS' + (dP o Gamma)^T Q - diag(beta gamma) dX S
//         + (dKK + dKK^T) K,     dKK = diag(beta) dA o Gamma
//   dV  = diag(beta) dX          (GLA: dV = dU)
// With split strengths (erase beta in E, write bw in f), bw replaces beta in X's
// V term and in dV, and <dX_t, V_t> is the write strength's gradient.
//   dA  = strict_lower(-dX U^T)  (because T (I + A) = I, -T^T dU X^T T^T = -dX U^T)
//   dbeta_t = <dX_t, V_t> + gamma_t <dRw_t, K_t> + sum_s dA_ts B_ts,  dRw = -dX S
//   dg_t    = gamma_t <(dO S)_t, Q_t> - e^{g_C-g_t} <(U dS')_t, K_t> + beta_t gamma_t <dRw_t, K_t>
//             + rows - columns of (dP o P) and of (dA o A),
//   dg_C   += gamma_C <dS', S> + sum_t e^{g_C-g_t} <(U dS')_t, K_t>,
// and d ln alpha_s = sum over t >= s in the chunk of dg_t.
//
// Three kernels:
//   bwd_states_kernel: the forward chunk recursion, storing the state entering
//     every chunk (one workgroup per head and 64-row value slice);
//   bwd_chunk_kernel: the chunks in reverse order, recomputing each chunk's
//     factors from its stored state and carrying dS in LDS; dv and dS0 rows
//     belong to the slice and are written in full, dq, dk, d ln alpha and dbeta
//     are sums over value rows and are written as per-slice partials;
//   bwd_reduce_kernel: the sum over slices and dalpha = d ln alpha / alpha.
// Products are 32x32 tiles on the float32 MFMA (v_mfma_f32_32x32x2f32).
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_f32.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;
constexpr int kC = 32;       // tokens per chunk
constexpr int kSL = 64;      // value rows per workgroup
constexpr int LV = kSL + 1;  // row stride of [32][64] value-row arrays
constexpr int LM = kC + 1;   // row stride of 32x32 matrices
constexpr int LB = kC + 4;   // row stride of the k-Gram (float4 rows for the solve)

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }

// accumulator element e of a 32x32 tile sits at row 8 (e / 4) + 4 kg + e % 4,
// column l32 (lane = 32 kg + l32)
__device__ __forceinline__ int acc_row(int e, int kg) { return 8 * (e >> 2) + 4 * kg + (e & 3); }

// Sum over the 32 lanes of each half-wave: quad and row steps on DPP, the
// lane ^ 16 step on v_permlane16_swap (a VALU exchange of the two 16-lane rows
// of each 32-lane group), not on the LDS-path swizzle.
__device__ __forceinline__ float sum32(float x) {
    x += dpp_move<0xB1>(x);   // lane ^ 1
    x += dpp_move<0x4E>(x);   // lane ^ 2
    x += dpp_move<0x141>(x);  // row half mirror
    x += dpp_move<0x140>(x);  // row mirror
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row sums of a tile: rows of the lane's half go to out[row] from lane l32 == 0.
__device__ __forceinline__ void store_row_sums(const f32x16& x, float* out, int l32, int kg, float sign) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float s = sum32(x[e]);
        if (l32 == 0) out[acc_row(e, kg)] = sign * s;
    }
}
// Column sums of a tile: out[column] from the lanes of half 0.
__device__ __forceinline__ void store_col_sums(const f32x16& x, float* out, int l32, int kg, float sign) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += x[e];
    s += __shfl_xor(s, 32, 64);
    if (kg == 0) out[l32] = sign * s;
}

// Chunk gates by wave 0 (lanes 0..31 hold tokens, with their alpha and the
// erase and write strengths already loaded): log2 cumulative decay G2,
// gamma = 2^G2, Dd = 2^(G2_C - G2), beta (erase), bw (write) and beta gamma;
// past T: identity tokens (alpha = 1, beta = 0).
template <bool GDN>
__device__ __forceinline__ void chunk_gates(float a_raw, float b_raw, float w_raw, int c0, int T, int lane,
                                            float* G2, float* gam, float* Dd, float* bet, float* bw, float* bg,
                                            float* gC) {
    const int t = lane & 31;
    const bool in = c0 + t < T;
    float la = in ? __log2f(a_raw) : 0.f;
    const float b = (GDN && in) ? b_raw : 0.f;
    const float bwv = (GDN && in) ? w_raw : 0.f;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
        const float y = __shfl_up(la, off, 32);
        if (t >= off) la += y;
    }
    const float last = __shfl(la, 31, 32);
    if (lane < 32) {
        const float g = __builtin_amdgcn_exp2f(la);
        G2[t] = la;
        gam[t] = g;
        Dd[t] = __builtin_amdgcn_exp2f(last - la);
        bet[t] = b;
        bw[t] = bwv;
        bg[t] = b * g;
        if (t == 0) *gC = __builtin_amdgcn_exp2f(last);
    }
}

// T = (I + diag(bet) B)^-1 for the strictly lower part of B (row stride LB, as
// float4 rows) into Tm (row stride LM), from its 16x16 blocks: the two diagonal
// blocks D0, D1 by forward substitution side by side (lane (b, c) of each
// half-wave owns column c of block b, x_r = [r == c] - bet_r sum_{j<r} B_rj x_j,
// rows read as float4 two rows ahead), then T10 = -D1 diag(bet) B10 D0 on the
// fp32 MFMA (16x16x4).  The upper right block of Tm stays zero from the start.
// All 64 lanes of the wave take part.
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
        for (int r = 0; r < 16; ++r) Tm[(16 * b + r) * LM + 16 * b + c] = x[r];
    }
    // T10 = -D1 (diag(bet) B10) D0: lane (n16, g4) supplies contraction indices
    // 4 g4 .. 4 g4 + 3 and holds rows 4 g4 .. 4 g4 + 3 of column n16
    const int n16 = lane & 15, g4 = lane >> 4;
    f32x4 y = {}, t10 = {};
    const f32x4 br10 = *reinterpret_cast<const f32x4*>(&Bm[(16 + n16) * LB + 4 * g4]);
    const float bs = bet[16 + n16];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) y = mfma4(br10[kk] * bs, Tm[(4 * g4 + kk) * LM + n16], y);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t10 = mfma4(Tm[(16 + n16) * LM + 16 + 4 * g4 + kk], y[kk], t10);
#pragma unroll
    for (int r = 0; r < 4; ++r) Tm[(16 + 4 * g4 + r) * LM + n16] = -t10[r];
}

// ---------------------------------------------------------------------------
// Forward states: S entering chunk n goes to ckpt[bh][n][rows of the slice].
template <int MODE, int DK, typename E>
__global__ __launch_bounds__(kThreads) void bwd_states_kernel(BwdJob J) {
    constexpr bool GDN = MODE == 0;
    constexpr int NJ = DK / 32;
    constexpr int L1 = DK + 1;
    __shared__ float Ks[kC * L1];
    __shared__ float Us[kC * LV];  // V, then X, then U
    __shared__ float Ss[kSL * L1];
    __shared__ __align__(16) float Bm[GDN ? kC * LB : 4];
    __shared__ float Tm[GDN ? kC * LM : 1];
    __shared__ float G2[kC], gam[kC], Dd[kC], bet[kC], bw[kC], bg[kC], gC[1];

    const int slices = J.dv / kSL;
    int bh, sl;
    unit_part(blockIdx.x, J.BH, slices, bh, sl);  // a head's slices share its input reads in L2
    const int r0 = sl * kSL;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, kg = lane >> 5;
    const int T = J.T, dv = J.dv;
    const E* k = static_cast<const E*>(J.k);
    const E* v = static_cast<const E*>(J.v);
    const size_t tok0 = (size_t)bh * T;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;
    auto row = [&](int e) { return acc_row(e, kg); };

    for (int x = tid; x < kSL * DK; x += kThreads) Ss[x / DK * L1 + x % DK] = J.S0 ? J.S0[s_base + x] : 0.f;
    if constexpr (GDN)
        for (int x = tid; x < kC * LM; x += kThreads) Tm[x] = 0.f;  // T's upper right block stays zero

    // The next chunk's k, v and gates are fetched into registers while this
    // chunk computes (unconditional loads from a clamped token index; masking
    // on the way into LDS), which hides HBM latency at one workgroup per CU.
    constexpr int NK = kC * DK / kThreads, NV = kC * kSL / kThreads;
    E pk[NK], pv[NV];
    float pa = 1.f, pb = 0.f, pw = 0.f;
    auto fetch = [&](int cn) {
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int x = tid + m * kThreads, t = min(cn + x / DK, T - 1);
            pk[m] = k[(tok0 + t) * DK + x % DK];
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreads, t = min(cn + x / kSL, T - 1);
            pv[m] = v[(tok0 + t) * dv + r0 + x % kSL];
        }
        if (w == 0) {
            const int t = min(cn + l32, T - 1);
            pa = J.alpha[tok0 + t];
            if (GDN) {
                pb = J.beta[tok0 + t];
                pw = J.beta_w[tok0 + t];
            }
        }
    };
    fetch(0);

    for (int n = 0; n < J.nchunks; ++n) {
        const int c0 = n * kC;
        __syncthreads();
        float4* ck4 = reinterpret_cast<float4*>(J.ckpt + (((size_t)bh * J.nchunks + n) * dv + r0) * DK);
#pragma unroll
        for (int m = 0; m < kSL * DK / 4 / kThreads; ++m) {
            const int x = 4 * (tid + m * kThreads);
            const float* src = Ss + x / DK * L1 + x % DK;
            ck4[tid + m * kThreads] = make_float4(src[0], src[1], src[2], src[3]);
        }
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int x = tid + m * kThreads, t = x / DK;
            Ks[t * L1 + x % DK] = c0 + t < T ? to_f32(pk[m]) : 0.f;
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreads, t = x / kSL;
            Us[t * LV + x % kSL] = c0 + t < T ? to_f32(pv[m]) : 0.f;
        }
        if (w == 0) chunk_gates<GDN>(pa, pb, pw, c0, T, lane, G2, gam, Dd, bet, bw, bg, gC);
        if (n + 1 < J.nchunks) fetch(c0 + kC);
        __syncthreads();
        if constexpr (GDN) {
            if (w == 0) {  // B = strict_lower(Gamma o K K^T)
                auto kr = [&](int s) { return Ks[l32 * L1 + 2 * s + kg]; };
                const f32x16 c = chain<DK / 2>(kr, kr, f32x16{});
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = row(e);
                    Bm[t * LB + l32] = l32 < t ? __builtin_amdgcn_exp2f(G2[t] - G2[l32]) * c[e] : 0.f;
                }
            } else if (w < 3) {  // X = beta V - beta gamma K S^T, value columns 32 (w - 1) ..
                const int I = w - 1;
                f32x16 c;
#pragma unroll
                for (int e = 0; e < 16; ++e) c[e] = bw[row(e)] * Us[row(e) * LV + 32 * I + l32];
                const float nbg = -bg[l32];
                c = chain<DK / 2>([&](int s) { return nbg * Ks[l32 * L1 + 2 * s + kg]; },
                                  [&](int s) { return Ss[(32 * I + l32) * L1 + 2 * s + kg]; }, c);
#pragma unroll
                for (int e = 0; e < 16; ++e) Us[row(e) * LV + 32 * I + l32] = c[e];
            }
            __syncthreads();
            if (w == 0) {  // T, then U = T X in place
                solve_unit_lower(Bm, bet, Tm, lane);
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    const f32x16 c = chain<kC / 2>([&](int s) { return Tm[l32 * LM + 2 * s + kg]; },
                                                   [&](int s) { return Us[(2 * s + kg) * LV + 32 * I + l32]; },
                                                   f32x16{});
#pragma unroll
                    for (int e = 0; e < 16; ++e) Us[row(e) * LV + 32 * I + l32] = c[e];
                }
            }
            __syncthreads();
        }
        // S <- gamma_C S + U^T diag(e^{g_C - g}) K
        for (int tile = w; tile < 2 * NJ; tile += 4) {
            const int I = tile / NJ, Jt = tile - I * NJ;
            f32x16 c;
#pragma unroll
            for (int e = 0; e < 16; ++e) c[e] = gC[0] * Ss[(32 * I + row(e)) * L1 + 32 * Jt + l32];
            c = chain<kC / 2>([&](int s) { return Us[(2 * s + kg) * LV + 32 * I + l32]; },
                              [&](int s) { return Dd[2 * s + kg] * Ks[(2 * s + kg) * L1 + 32 * Jt + l32]; }, c);
#pragma unroll
            for (int e = 0; e < 16; ++e) Ss[(32 * I + row(e)) * L1 + 32 * Jt + l32] = c[e];
        }
    }
}

// ---------------------------------------------------------------------------
// The reverse chunk pass.
template <int MODE, int DK, typename E>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_chunk_kernel(
    BwdJob J) {
    constexpr bool GDN = MODE == 0;
    constexpr int NJ = DK / 32;  // key-column tiles: wave w < NJ owns dq and dk tile w
    constexpr int L1 = DK + 1;
    __shared__ float Qs[kC * L1];
    __shared__ float Ks[kC * L1];
    __shared__ float Ss[kSL * L1];   // state entering the chunk
    __shared__ float dSs[kSL * L1];  // gradient at the state leaving it, then entering it
    __shared__ float Vs[kC * LV];    // V, then dX
    __shared__ float dOs[kC * LV];
    __shared__ float Us[kC * LV];    // V, then X, then U
    __shared__ float dUs[kC * LV];
    __shared__ __align__(16) float Bm[GDN ? kC * LB : 4];
    __shared__ float Pm[kC * LM];
    __shared__ float Tm[GDN ? kC * LM : 1];
    __shared__ float dQKm[kC * LM];  // dP o Gamma
    __shared__ float dKKm[GDN ? kC * LM : 1];
    __shared__ float G2[kC], gam[kC], Dd[kC], bet[kC], bw[kC], bg[kC], gC[1];
    __shared__ float dgp[16 * kC];   // per-product contributions to dg (fixed slots)
    __shared__ float dbp[8 * kC];    // ... to dbeta
    __shared__ float dgc[16];        // ... to dg_C

    const int slices = J.dv / kSL;
    int bh, slice;
    unit_part(blockIdx.x, J.BH, slices, bh, slice);  // a head's slices share its input reads in L2
    const int r0 = slice * kSL;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, kg = lane >> 5;
    const int T = J.T, dv = J.dv;
    const E* q = static_cast<const E*>(J.q);
    const E* k = static_cast<const E*>(J.k);
    const E* v = static_cast<const E*>(J.v);
    const E* dO = static_cast<const E*>(J.dO);
    const size_t tok0 = (size_t)bh * T;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;
    const size_t part_tok = ((size_t)slice * J.BH + bh) * T;  // this slice's partial rows
    float* pdq = J.part;
    float* pdk = pdq + (size_t)slices * J.BH * T * DK;
    float* pdl = pdk + (size_t)slices * J.BH * T * DK;
    float* pdb = pdl + (size_t)slices * J.BH * T;
    float* pdbw = pdb + (size_t)slices * J.BH * T;  // write strengths (split strengths only)
    auto row = [&](int e) { return acc_row(e, kg); };

    for (int x = tid; x < kSL * DK; x += kThreads) dSs[x / DK * L1 + x % DK] = J.dST ? J.dST[s_base + x] : 0.f;
    if constexpr (GDN)
        for (int x = tid; x < kC * LM; x += kThreads) Tm[x] = 0.f;  // T's upper right block stays zero

    // The next chunk's (in reverse order) q, k, v, dO and gates are fetched
    // into registers during this one's last two phases (unconditional loads
    // from a clamped token index; masking on the way into LDS).  Issued
    // earlier, the registers would be live through the phases with the most
    // accumulators.  Its stored state, 32 more registers per lane, is read at
    // the chunk's start instead: prefetched, it made the kernel spill more and
    // ran slower.
    constexpr int NK = kC * DK / kThreads, NV = kC * kSL / kThreads;
    E pq[NK], pk[NK], pv[NV], pd[NV];
    float pa = 1.f, pb = 0.f, pw = 0.f;
    auto fetch = [&](int n) {
        const int cn = n * kC;
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int x = tid + m * kThreads, t = min(cn + x / DK, T - 1);
            const size_t gi = (tok0 + t) * DK + x % DK;
            pq[m] = q[gi];
            pk[m] = k[gi];
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreads, t = min(cn + x / kSL, T - 1);
            const size_t gi = (tok0 + t) * dv + r0 + x % kSL;
            pv[m] = v[gi];
            pd[m] = dO ? dO[gi] : E(0);
        }
        if (w == 0) {
            const int t = min(cn + l32, T - 1);
            pa = J.alpha[tok0 + t];
            if (GDN) {
                pb = J.beta[tok0 + t];
                pw = J.beta_w[tok0 + t];
            }
        }
    };
    fetch(J.nchunks - 1);

    for (int n = J.nchunks - 1; n >= 0; --n) {
        const int c0 = n * kC;
        __syncthreads();  // the previous chunk is done with every array
        {  // the stored state: all of a thread's 16-byte loads are issued before any is used
            constexpr int NS4 = kSL * DK / 4 / kThreads;
            const float4* ck4 =
                reinterpret_cast<const float4*>(J.ckpt + (((size_t)bh * J.nchunks + n) * dv + r0) * DK);
            float4 sv[NS4];
#pragma unroll
            for (int m = 0; m < NS4; ++m) sv[m] = ck4[tid + m * kThreads];
#pragma unroll
            for (int m = 0; m < NS4; ++m) {
                const int x = 4 * (tid + m * kThreads);
                float* dst = Ss + x / DK * L1 + x % DK;
                dst[0] = sv[m].x;
                dst[1] = sv[m].y;
                dst[2] = sv[m].z;
                dst[3] = sv[m].w;
            }
        }
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int x = tid + m * kThreads, t = x / DK, y = t * L1 + x % DK;
            const bool in = c0 + t < T;
            Qs[y] = in ? to_f32(pq[m]) : 0.f;
            Ks[y] = in ? to_f32(pk[m]) : 0.f;
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreads, t = x / kSL, y = t * LV + x % kSL;
            const bool in = c0 + t < T;
            const float vv = in ? to_f32(pv[m]) : 0.f;
            Vs[y] = vv;
            Us[y] = vv;
            dOs[y] = in ? to_f32(pd[m]) : 0.f;
        }
        for (int x = tid; x < 16 * kC; x += kThreads) dgp[x] = 0.f;
        for (int x = tid; x < 8 * kC; x += kThreads) dbp[x] = 0.f;
        if (tid < 16) dgc[tid] = 0.f;
        if (w == 0) chunk_gates<GDN>(pa, pb, pw, c0, T, lane, G2, gam, Dd, bet, bw, bg, gC);
        __syncthreads();

        f32x16 accQ = {}, accK = {};
        f32x16 ksT = {};  // waves 2, 3 (delta rule): (K S^T)^T on value columns 32 (w - 2) .., kept to phase 5
        // Phase 1: B, P, X; the owners start dQ = diag(gamma) dO S (+ its dg share)
        if (GDN && w == 0) {
            auto kr = [&](int s) { return Ks[l32 * L1 + 2 * s + kg]; };
            const f32x16 c = chain<DK / 2>(kr, kr, f32x16{});
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                Bm[t * LB + l32] = l32 < t ? __builtin_amdgcn_exp2f(G2[t] - G2[l32]) * c[e] : 0.f;
            }
        } else if (w == 1) {
            const f32x16 c = chain<DK / 2>([&](int s) { return Qs[l32 * L1 + 2 * s + kg]; },
                                           [&](int s) { return Ks[l32 * L1 + 2 * s + kg]; }, f32x16{});
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                Pm[t * LM + l32] = l32 <= t ? __builtin_amdgcn_exp2f(G2[t] - G2[l32]) * c[e] : 0.f;
            }
        } else if (GDN && w >= 2) {
            const int I = w - 2;
            // (K S^T)^T = S K^T with the token along the lanes: X_t = beta_t V_t - beta_t gamma_t (K S^T)_t
            // is written row by row, and the tile serves <dX_t, (K S^T)_t> in phase 5 as an in-lane sum
            ksT = chain<DK / 2>([&](int s) { return Ss[(32 * I + l32) * L1 + 2 * s + kg]; },
                                [&](int s) { return Ks[l32 * L1 + 2 * s + kg]; }, f32x16{});
            const float b = bw[l32], nbg = -bg[l32];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int y = l32 * LV + 32 * I + row(e);
                Us[y] = b * Us[y] + nbg * ksT[e];
            }
        } else if (!GDN && w >= 2) {  // GLA: dU = Kd dS'^T starts here
            const int I = w - 2;
            const float dd = Dd[l32];
            const f32x16 c = chain<DK / 2>([&](int s) { return dd * Ks[l32 * L1 + 2 * s + kg]; },
                                           [&](int s) { return dSs[(32 * I + l32) * L1 + 2 * s + kg]; }, f32x16{});
#pragma unroll
            for (int e = 0; e < 16; ++e) dUs[row(e) * LV + 32 * I + l32] = c[e];
        }
        if (w < NJ) {
            const float gl = gam[l32];
            accQ = chain<kSL / 2>([&](int s) { return gl * dOs[l32 * LV + 2 * s + kg]; },
                                  [&](int s) { return Ss[(2 * s + kg) * L1 + 32 * w + l32]; }, accQ);
            f32x16 x;
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = accQ[e] * Qs[row(e) * L1 + 32 * w + l32];
            store_row_sums(x, dgp + w * kC, l32, kg, 1.f);  // dg slots 0..3
        }
        __syncthreads();
        // Phase 2 (delta rule): T and U = T X; dU = Kd dS'^T
        if constexpr (GDN) {
            if (w == 0) {
                solve_unit_lower(Bm, bet, Tm, lane);
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    const f32x16 c = chain<kC / 2>([&](int s) { return Tm[l32 * LM + 2 * s + kg]; },
                                                   [&](int s) { return Us[(2 * s + kg) * LV + 32 * I + l32]; },
                                                   f32x16{});
#pragma unroll
                    for (int e = 0; e < 16; ++e) Us[row(e) * LV + 32 * I + l32] = c[e];
                }
            } else if (w < 3) {
                const int I = w - 1;
                const float dd = Dd[l32];
                const f32x16 c = chain<DK / 2>([&](int s) { return dd * Ks[l32 * L1 + 2 * s + kg]; },
                                               [&](int s) { return dSs[(32 * I + l32) * L1 + 2 * s + kg]; },
                                               f32x16{});
#pragma unroll
                for (int e = 0; e < 16; ++e) dUs[row(e) * LV + 32 * I + l32] = c[e];
            }
            __syncthreads();
        }
        // Phase 3: dP (waves 0 and 3 both form it: wave 0 writes dP * Gamma, wave 3 the
        // row and column sums of dP * P), dU += P^T dO (waves 1, 2), the owners' dK += Kd-part
        if (w == 0 || w == 3) {
            const f32x16 c = chain<kSL / 2>([&](int s) { return dOs[l32 * LV + 2 * s + kg]; },
                                            [&](int s) { return Us[l32 * LV + 2 * s + kg]; }, f32x16{});
            if (w == 0) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = row(e);
                    dQKm[t * LM + l32] = l32 <= t ? c[e] * __builtin_amdgcn_exp2f(G2[t] - G2[l32]) : 0.f;
                }
            } else {
                f32x16 L;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = row(e);
                    L[e] = l32 <= t ? c[e] * Pm[t * LM + l32] : 0.f;
                }
                store_row_sums(L, dgp + 8 * kC, l32, kg, 1.f);   // dg slot 8
                store_col_sums(L, dgp + 9 * kC, l32, kg, -1.f);  // dg slot 9
            }
        } else if (w < 3) {
            const int I = w - 1;
            {  // e^{g_C - g_t} <(U dS')_t, K_t> = <U_t, dU_t> while dU holds Kd dS'^T: lane l32 takes
               // token l32, each half 16 of the tile's value columns
                float t1 = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int y = l32 * LV + 32 * I + 16 * kg + i;
                    t1 += Us[y] * dUs[y];
                }
                t1 += __shfl_xor(t1, 32, 64);
                if (kg == 0) dgp[(4 + I) * kC + l32] = -t1;  // dg slots 4, 5
            }
            f32x16 c;
#pragma unroll
            for (int e = 0; e < 16; ++e) c[e] = dUs[row(e) * LV + 32 * I + l32];
            c = chain<kC / 2>([&](int s) { return Pm[(2 * s + kg) * LM + l32]; },
                              [&](int s) { return dOs[(2 * s + kg) * LV + 32 * I + l32]; }, c);
#pragma unroll
            for (int e = 0; e < 16; ++e) dUs[row(e) * LV + 32 * I + l32] = c[e];
        }
        if (w < NJ) {  // dKd = U dS'
            const f32x16 c = chain<kSL / 2>([&](int s) { return Us[l32 * LV + 2 * s + kg]; },
                                            [&](int s) { return dSs[(2 * s + kg) * L1 + 32 * w + l32]; }, f32x16{});
#pragma unroll
            for (int e = 0; e < 16; ++e) accK[e] += Dd[row(e)] * c[e];
        }
        __syncthreads();
        // Phase 4: dX = T^T dU (delta rule; computed as dX^T = dU^T T, the token along the lanes, so
        // <dX_t, V_t> is an in-lane sum; dX replaces V row by row); the owners' dQ, dK += dQK parts
        if (GDN && (w == 1 || w == 2)) {
            const int I = w - 1;
            const f32x16 c = chain<kC / 2>([&](int s) { return dUs[(2 * s + kg) * LV + 32 * I + l32]; },
                                           [&](int s) { return Tm[(2 * s + kg) * LM + l32]; }, f32x16{});
            float db = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int y = l32 * LV + 32 * I + row(e);
                db += c[e] * Vs[y];
                Vs[y] = c[e];
            }
            db += __shfl_xor(db, 32, 64);
            if (kg == 0) dbp[I * kC + l32] = db;  // dbeta slots 0, 1
        }
        if (w == 0 || w == 3) {  // dO's last reader is the dS update: scale its rows by gamma in place
            for (int x = (w == 0 ? 0 : 64) + lane; x < kC * kSL; x += 128) {
                const int t = x / kSL;
                dOs[t * LV + x - t * kSL] *= gam[t];
            }
        }
        if (w < NJ) {
            accQ = chain<kC / 2>([&](int s) { return dQKm[l32 * LM + 2 * s + kg]; },
                                 [&](int s) { return Ks[(2 * s + kg) * L1 + 32 * w + l32]; }, accQ);
            accK = chain<kC / 2>([&](int s) { return dQKm[(2 * s + kg) * LM + l32]; },
                                 [&](int s) { return Qs[(2 * s + kg) * L1 + 32 * w + l32]; }, accK);
        }
        __syncthreads();
        // the next chunk's inputs are in flight through phases 5 and 6
        if (n > 0) fetch(n - 1);
        // Phase 5: dA (waves 0 and 1 both form it: wave 0 writes dKK, wave 1 the sums),
        // dRw (owners), dS
        if constexpr (GDN) {
            if (w < 2) {
                const f32x16 c = chain<kSL / 2>([&](int s) { return -Vs[l32 * LV + 2 * s + kg]; },
                                                [&](int s) { return Us[l32 * LV + 2 * s + kg]; }, f32x16{});
                if (w == 0) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = row(e);
                        dKKm[t * LM + l32] = l32 < t ? bet[t] * c[e] * __builtin_amdgcn_exp2f(G2[t] - G2[l32]) : 0.f;
                    }
                } else {
                    f32x16 xb, xa;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = row(e);
                        const float da = l32 < t ? c[e] : 0.f;
                        const float b = Bm[t * LB + l32];
                        xb[e] = da * b;
                        xa[e] = da * bet[t] * b;
                    }
                    store_row_sums(xb, dbp + 6 * kC, l32, kg, 1.f);    // dbeta slot 6 (dg: beta_t times it)
                    store_col_sums(xa, dgp + 15 * kC, l32, kg, -1.f);  // dg slot 15
                }
            }
            if (w >= 2) {  // <dRw_t, K_t> = -<dX_t, (K S^T)_t> over this wave's value columns
                const int I = w - 2;
                float wt = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) wt += ksT[e] * Vs[l32 * LV + 32 * I + row(e)];
                wt = -(wt + __shfl_xor(wt, 32, 64));
                if (kg == 0) {
                    dbp[(2 + I) * kC + l32] = gam[l32] * wt;  // dbeta slots 2, 3
                    dgp[(10 + I) * kC + l32] = bg[l32] * wt;  // dg slots 10, 11
                }
            }
            if (w < NJ) {  // dRw = -dX S
                const f32x16 c = chain<kSL / 2>([&](int s) { return -Vs[l32 * LV + 2 * s + kg]; },
                                                [&](int s) { return Ss[(2 * s + kg) * L1 + 32 * w + l32]; },
                                                f32x16{});
#pragma unroll
                for (int e = 0; e < 16; ++e) accK[e] += bg[row(e)] * c[e];
            }
        }
        // dV = diag(bw) dX (delta rule) or dU (linear attention), row-major from LDS
        for (int x = tid; x < kC * kSL; x += kThreads) {
            const int t = x / kSL, i = x % kSL;
            if (c0 + t < T)
                J.dv_out[(tok0 + c0 + t) * dv + r0 + i] = GDN ? bw[t] * Vs[t * LV + i] : dUs[t * LV + i];
        }
        // dS = gamma_C dS' + dO^T diag(gamma) Q - dX^T diag(beta gamma) K, and <dS', S>
        for (int tile = w; tile < 2 * NJ; tile += 4) {
            const int I = tile / NJ, Jt = tile - I * NJ;
            f32x16 c;
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int y = (32 * I + row(e)) * L1 + 32 * Jt + l32;
                const float d = dSs[y];
                ss += d * Ss[y];
                c[e] = gC[0] * d;
            }
            // the two products as one chain over 2 C (GDN) or C tokens
            constexpr int H2 = kC / 2;
            c = chain<GDN ? kC : H2>(
                [&](int s) {
                    const int t = 2 * (s % H2) + kg;
                    return s < H2 ? dOs[t * LV + 32 * I + l32] : -Vs[t * LV + 32 * I + l32];
                },
                [&](int s) {
                    const int t = 2 * (s % H2) + kg;
                    return s < H2 ? Qs[t * L1 + 32 * Jt + l32] : bg[t] * Ks[t * L1 + 32 * Jt + l32];
                },
                c);
#pragma unroll
            for (int e = 0; e < 16; ++e) dSs[(32 * I + row(e)) * L1 + 32 * Jt + l32] = c[e];
            ss = group_sum<64>(ss);
            if (lane == 0) dgc[4 + tile] = ss;
        }
        __syncthreads();
        // Phase 6: dK += (dKK + dKK^T) K; partial dq, dk; dg -> d ln alpha, dbeta
        if (w < NJ) {
            if constexpr (GDN)
                accK = chain<kC / 2>(
                    [&](int s) { return dKKm[l32 * LM + 2 * s + kg] + dKKm[(2 * s + kg) * LM + l32]; },
                    [&](int s) { return Ks[(2 * s + kg) * L1 + 32 * w + l32]; }, accK);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                if (c0 + t < T) {
                    const size_t o = (part_tok + c0 + t) * DK + 32 * w + l32;
                    pdq[o] = accQ[e];
                    pdk[o] = accK[e];
                }
            }
        }
        if (w == 3) {
            // one wave (lanes 0..31 hold tokens) sums the slots in a fixed order
            const int t = l32;
            float dg = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) dg += dgp[s * kC + t];
            if constexpr (GDN) dg += bet[t] * dbp[6 * kC + t];  // the rows of dA o A
            // d g_C: gamma_C <dS', S> and the sum over tokens of e^{g_C - g_t} <(U dS')_t, K_t>
            const float t1 = group_sum<32>(dgp[4 * kC + t] + dgp[5 * kC + t]);
            if (t == kC - 1) {
                float sc = 0.f;
#pragma unroll
                for (int s = 4; s < 12; ++s) sc += dgc[s];
                dg += gC[0] * sc - t1;
            }
            // reverse cumulative sum over the chunk: d ln alpha_s = sum_{t >= s} dg_t
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                const float y = __shfl_down(dg, off, 32);
                if (t + off < 32) dg += y;
            }
            // dbeta slots 0, 1 belong to the write strength (they come from V), the rest to the erase one
            const float dbw = dbp[t] + dbp[kC + t];
            float dbe = 0.f;
#pragma unroll
            for (int s = 2; s < 8; ++s) dbe += dbp[s * kC + t];
            if (kg == 0 && c0 + t < T) {
                pdl[part_tok + c0 + t] = dg;
                if (J.dbeta_w) {
                    pdb[part_tok + c0 + t] = dbe;
                    pdbw[part_tok + c0 + t] = dbw;
                } else {
                    pdb[part_tok + c0 + t] = dbe + dbw;
                }
            }
        }
    }
    __syncthreads();
    for (int x = tid; x < kSL * DK; x += kThreads) J.dS0[s_base + x] = dSs[x / DK * L1 + x % DK];
}

// Sum of the per-slice partials; dalpha = d ln alpha / alpha.
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(BwdJob J) {
    const size_t n_tok = (size_t)J.BH * J.T;
    const size_t n_el = n_tok * J.dk;
    const int slices = J.dv / kSL;
    const float* pdq = J.part;
    const float* pdk = pdq + (size_t)slices * n_el;
    const float* pdl = pdk + (size_t)slices * n_el;
    const float* pdb = pdl + (size_t)slices * n_tok;
    const float* pdbw = pdb + (size_t)slices * n_tok;
    for (size_t x = (size_t)blockIdx.x * kThreads + threadIdx.x; x < n_el; x += (size_t)gridDim.x * kThreads) {
        float a = 0.f, b = 0.f;
        for (int s = 0; s < slices; ++s) {
            a += pdq[s * n_el + x];
            b += pdk[s * n_el + x];
        }
        J.dq[x] = a;
        J.dk_out[x] = b;
        if (x % J.dk == 0) {
            const size_t tk = x / J.dk;
            float l = 0.f, d = 0.f, dw = 0.f;
            for (int s = 0; s < slices; ++s) {
                l += pdl[s * n_tok + tk];
                d += pdb[s * n_tok + tk];
                if (J.dbeta_w) dw += pdbw[s * n_tok + tk];
            }
            J.dalpha[tk] = l / J.alpha[tk];
            if (J.dbeta) J.dbeta[tk] = d;
            if (J.dbeta_w) J.dbeta_w[tk] = dw;
        }
    }
}

template <int MODE, int DK, typename E>
hipError_t launch_typed(const BwdJob& J, hipStream_t s) {
    const dim3 grid((unsigned)((size_t)J.BH * (J.dv / kSL)));
    hipLaunchKernelGGL((bwd_states_kernel<MODE, DK, E>), grid, dim3(kThreads), 0, s, J);
    hipLaunchKernelGGL((bwd_chunk_kernel<MODE, DK, E>), grid, dim3(kThreads), 0, s, J);
    const size_t n_el = (size_t)J.BH * J.T * J.dk;
    const size_t want = (n_el + kThreads - 1) / kThreads;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(blocks), dim3(kThreads), 0, s, J);
    return hipGetLastError();
}

template <int MODE, typename E>
hipError_t launch_mode(const BwdJob& J, hipStream_t s) {
    switch (J.dk) {
        case 32: return launch_typed<MODE, 32, E>(J, s);
        case 64: return launch_typed<MODE, 64, E>(J, s);
        case 128: return launch_typed<MODE, 128, E>(J, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool scan_bwd_supported(int dk, int dv) {
    return (dk == 32 || dk == 64 || dk == 128) && dv >= kSL && dv % kSL == 0 && dv <= 4096;
}

size_t scan_bwd_workspace_floats(int BH, int T, int dk, int dv) {
    const size_t nchunks = ((size_t)T + kC - 1) / kC;
    const size_t slices = (size_t)dv / kSL;
    return (size_t)BH * nchunks * dv * dk + slices * BH * T * (2 * (size_t)dk + 3);
}

hipError_t launch_scan_bwd(int mode, int dtype, BwdJob J, hipStream_t s) {
    J.nchunks = (J.T + kC - 1) / kC;
    J.part = J.ckpt + (size_t)J.BH * J.nchunks * J.dv * J.dk;
    if (dtype == 0)
        return mode == 0 ? launch_mode<0, float>(J, s) : launch_mode<1, float>(J, s);
    return mode == 0 ? launch_mode<0, uint16_t>(J, s) : launch_mode<1, uint16_t>(J, s);
}

}  // namespace gds
