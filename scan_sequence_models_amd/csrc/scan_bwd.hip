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
//     are sums over value rows: with one or two slices they go straight into the
//     outputs (two slices add onto zeros written by the states pass, with float
//     atomics: a + b = b + a, so the result does not depend on their order),
//     with more as per-slice partials;
//   bwd_reduce_kernel (more than two slices): the sum over slices and
//     dalpha = d ln alpha / alpha; bwd_finish_kernel (else): the division.
// Products are 32x32 tiles: in split bf16 on the bf16 MFMA for bf16 data, on
// the float32 MFMA for float32 data, their operands read from LDS eight k at a
// time (chain8_t).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_f32.hpp"
#include "solve.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;
constexpr int kThreadsR = 512;  // the reverse chunk pass: 8 waves, two per SIMD
// the states pass: 8 waves (two per SIMD) with bf16 data, 4 with float32 data
// (whose wider prefetch registers would spill at two waves per SIMD)
template <typename E>
constexpr int states_waves() { return std::is_same<E, uint16_t>::value ? 8 : 4; }
constexpr int kC = 32;       // tokens per chunk
constexpr int kSL = 64;      // value rows per workgroup
constexpr int LV = kSL + 1;  // row stride of [32][64] value-row arrays
constexpr int LB = kC + 4;   // row stride of the k-Gram (float4 rows for the solve)

// The elements of a 16-byte load: eight bf16 or four floats.
template <int EV>
__device__ __forceinline__ void unpack16(const uint4& u, float (&f)[EV]) {
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
    if constexpr (EV == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(wd[i] << 16);
            f[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(wd[i]);
    }
}

// accumulator element e of a 32x32 tile sits at row 8 (e / 4) + 4 kg + e % 4,
// column l32 (lane = 32 kg + l32)
__device__ __forceinline__ int acc_row(int e, int kg) { return 8 * (e >> 2) + 4 * kg + (e & 3); }
// p[acc_row(e, kg)] for e = 0 .. 15 from a 16-byte aligned per-token array: the
// rows of a lane come in four runs of four consecutive tokens, one 16-byte read each
__device__ __forceinline__ f32x16 acc_rows16(const float* p, int kg) {
    f32x16 r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&p[8 * b + 4 * kg]);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[4 * b + i] = v[i];
    }
    return r;
}

// Row sums of a tile: rows of the lane's half go to out[row].  A transposing
// butterfly over the 32 lanes of the half: at each step the two lanes of a pair
// (the two 16-lane rows, then the mirrors within a row, half-row and quad) each
// keep one half of their remaining elements and add the partner's copy of it,
// so 16 elements take 8 + 4 + 2 + 1 exchanges (and one more to finish) instead
// of 5 per element.  Lane l32 ends with element (l32 >> 1) of its row group.
__device__ __forceinline__ void store_row_sums(const f32x16& x, float* out, int l32, int kg, float sign) {
    // lane ^ 16: the lanes of 16-lane row 0 keep elements 0 .. 7, those of row 1
    // elements 8 .. 15 (v_permlane16_swap exchanges row 1 of its first operand with
    // row 0 of its second)
    float u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j + 8]), false, false);
        u[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool b3 = (l32 & 8) != 0, b2 = (l32 & 4) != 0, b1 = (l32 & 2) != 0;
    float t4[4], t2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // row mirror: lanes 0 .. 7 with 8 .. 15
        const float keep = b3 ? u[j + 4] : u[j], send = b3 ? u[j] : u[j + 4];
        t4[j] = keep + dpp_move<0x140>(send);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // half-row mirror: lanes 0 .. 3 with 4 .. 7
        const float keep = b2 ? t4[j + 2] : t4[j], send = b2 ? t4[j] : t4[j + 2];
        t2[j] = keep + dpp_move<0x141>(send);
    }
    float t1;
    {  // lane ^ 2
        const float keep = b1 ? t2[1] : t2[0], send = b1 ? t2[0] : t2[1];
        t1 = keep + dpp_move<0x4E>(send);
    }
    t1 += dpp_move<0xB1>(t1);  // lane ^ 1
    if ((l32 & 1) == 0) out[acc_row((l32 >> 1) & 15, kg)] = sign * t1;
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


// ---------------------------------------------------------------------------
// Forward states: S entering chunk n goes to ckpt[bh][n][rows of the slice].
//
// Only X = beta V - beta gamma K S^T, U = T X and the update of S depend on the
// state, so they alone make the serial chain; the rest runs ahead of it on the
// waves the chain leaves idle.  Eight waves (two per SIMD) with bf16 data, four
// with float32 data.  In the loop over chunks n (three barriers):
//   1: waves 1, 2 form X(n); wave 0 solves T(n + 1) from its k-Gram; wave 4 (wave
//      0 with four waves; two value slices) zeroes the outputs the reverse pass
//      adds into; wave 3 moves k(n + 2) and v(n + 1) from its registers into LDS,
//      forms the gates of chunk n + 2 and fetches k(n + 3) and v(n + 2) from HBM;
//   2: waves 1, 2 form U(n) = T(n) X(n); wave 3 forms the k-Gram of chunk n + 2;
//      waves 4 .. 7 store S entering chunk n, a quarter each (four waves: wave 0
//      half, waves 1, 2 a quarter each);
//   3: all waves update S, each on the tiles it keeps in registers.
// k and the gates are held three chunks deep, v/U, T and the k-Gram two.
// GLA (U = V, nothing to solve): wave 3 moves k(n + 1) and v(n + 1), wave 0
// zeroes the outputs (wave 3 with four waves) and waves 4 .. 7 store the state
// (wave 0 with four waves); a barrier; the update.
struct alignas(16) ChunkGatesLds {  // every array 16-byte aligned (kC floats each)
    float G2[kC], gam[kC], Dd[kC], bet[kC], bw[kC], bg[kC], gC[1];
};

template <int MODE, int DK, typename E>
__global__ __launch_bounds__(64 * states_waves<E>())
__attribute__((amdgpu_waves_per_eu(states_waves<E>() / 4, states_waves<E>() / 4))) void bwd_states_kernel(
    BwdJob J) {
    constexpr bool GDN = MODE == 0;
    // bf16 data: the products in split bf16 (about 16 significant bits each)
    constexpr bool SPLIT = std::is_same<E, uint16_t>::value;
    constexpr int NJ = DK / 32;
    constexpr int NW = states_waves<E>(), NTH = 64 * NW;
    // the wave that stages v: with eight waves and the delta rule, one whose X phase is short
    constexpr int VW = (GDN && NW == 8) ? 5 : 3;
    // Row strides: 16-byte rows (vector reads and writes along a row), and
    // k-operands read down a column as rows r and r + 8 (the two lane halves)
    // land 32 banks apart.
    constexpr int L1 = DK + 4, LU = kSL + 4, LT = kC + 4;
    constexpr int NB = GDN ? 3 : 2;  // k and gate buffers
    __shared__ __align__(16) float Ks[NB][kC * L1];
    __shared__ __align__(16) float Us[2][kC * LU];  // v, then X, then diag(e^{g_C - g}) U
    __shared__ __align__(16) float Ss[kSL * L1];
    __shared__ __align__(16) float Bm[GDN ? 2 : 1][GDN ? kC * LB : 4];
    __shared__ __align__(16) float Tm[GDN ? 2 : 1][GDN ? kC * LT : 1];
    __shared__ ChunkGatesLds gt[NB];

    const int slices = J.dv / kSL;
    int bh, sl;
    unit_part(blockIdx.x, J.BH, slices, bh, sl);  // a head's slices share its input reads in L2
    const int r0 = sl * kSL;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, kg = lane >> 5;
    const int T = J.T, dv = J.dv, NC = J.nchunks;
    const E* k = static_cast<const E*>(J.k);
    const E* v = static_cast<const E*>(J.v);
    const size_t tok0 = (size_t)bh * T;
    const size_t s_base = ((size_t)bh * dv + r0) * DK;
    auto row = [&](int e) { return acc_row(e, kg); };

    // Wave 3's inputs: a chunk of k or v in 16-byte loads from a token index
    // clamped into the sequence (unconditional; tokens past T are masked on the
    // way into LDS), the gates' inputs of a k chunk in lanes 0..31 (and 32..63).
    constexpr int EV = 16 / (int)sizeof(E);  // elements per load
    constexpr int RK = DK / EV, RV = kSL / EV;  // loads per row
    constexpr int FK = kC * RK / 64, FV = kC * RV / 64;
    uint4 rk[FK], rv[FV];
    float ra = 1.f, rb = 0.f, rw = 0.f;
    auto fetch_k = [&](int cn) {
#pragma unroll
        for (int m = 0; m < FK; ++m) {
            const int x = lane + 64 * m, t = min(cn * kC + x / RK, T - 1);
            rk[m] = *reinterpret_cast<const uint4*>(k + (tok0 + t) * DK + (x % RK) * EV);
        }
        const int t = min(cn * kC + l32, T - 1);
        ra = J.alpha[tok0 + t];
        if (GDN) {
            rb = J.beta[tok0 + t];
            rw = J.beta_w[tok0 + t];
        }
    };
    auto fetch_v = [&](int cn) {
#pragma unroll
        for (int m = 0; m < FV; ++m) {
            const int x = lane + 64 * m, t = min(cn * kC + x / RV, T - 1);
            rv[m] = *reinterpret_cast<const uint4*>(v + (tok0 + t) * dv + r0 + (x % RV) * EV);
        }
    };
    // k chunk cn into its buffer, and its gates
    auto put_k = [&](int cn) {
        float* dst = Ks[cn % NB];
#pragma unroll
        for (int m = 0; m < FK; ++m) {
            const int x = lane + 64 * m, t = x / RK;
            float f[EV];
            unpack16(rk[m], f);
            const bool in = cn * kC + t < T;
#pragma unroll
            for (int i = 0; i < EV; i += 4)
                *reinterpret_cast<f32x4*>(&dst[t * L1 + (x % RK) * EV + i]) =
                    in ? f32x4{f[i], f[i + 1], f[i + 2], f[i + 3]} : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        ChunkGatesLds& g = gt[cn % NB];
        chunk_gates<GDN>(ra, rb, rw, cn * kC, T, lane, g.G2, g.gam, g.Dd, g.bet, g.bw, g.bg, g.gC);
    };
    // v chunk cn into its buffer (GLA: as diag(e^{g_C - g}) V, gates of cn formed)
    auto put_v = [&](int cn) {
        float* dst = Us[cn & 1];
        const float* Dd = gt[cn % NB].Dd;
#pragma unroll
        for (int m = 0; m < FV; ++m) {
            const int x = lane + 64 * m, t = x / RV;
            float f[EV];
            unpack16(rv[m], f);
            const bool in = cn * kC + t < T;
            const float sc = in ? (GDN ? 1.f : Dd[t]) : 0.f;
#pragma unroll
            for (int i = 0; i < EV; i += 4)
                *reinterpret_cast<f32x4*>(&dst[t * LU + (x % RV) * EV + i]) =
                    sc * f32x4{f[i], f[i + 1], f[i + 2], f[i + 3]};
        }
    };
    // B(cn) = strict_lower(Gamma o K K^T) into its buffer
    auto k_gram = [&](int cn) {
        const float* Kb = Ks[cn % NB];
        const float* G2 = gt[cn % NB].G2;
        auto kr = [&](int i) { return lds_f32x8(&Kb[l32 * L1 + 16 * i + 8 * kg]); };
        const f32x16 c = chain8_t<SPLIT, DK / 16, true, true>(kr, kr, f32x16{});
        float* B = Bm[cn & 1];
        const f32x16 gt16 = acc_rows16(G2, kg);
        const float gs = G2[l32];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int t = row(e);
            B[t * LB + l32] = l32 < t ? __builtin_amdgcn_exp2f(gt16[e] - gs) * c[e] : 0.f;
        }
    };
    // the state entering chunk cn, from Ss: 16-byte pieces m0, m0 + 1, .. < m1
    // of each lane (kSL DK / 256 in all).  With rows of 64 floats or more the
    // 16-byte units of row r are stored XOR-permuted by r mod 16, the layout
    // the reverse pass reads them into LDS with.
    auto stash = [&](int cn, auto m0, auto m1) {
        f32x4* ck4 = reinterpret_cast<f32x4*>(J.ckpt + (((size_t)bh * NC + cn) * dv + r0) * DK);
#pragma unroll
        for (int m = decltype(m0)::value; m < decltype(m1)::value; ++m) {
            const int x = lane + 64 * m, r = x / (DK / 4), u = x % (DK / 4);
            ck4[x] = *reinterpret_cast<const f32x4*>(Ss + r * L1 + 4 * (DK >= 64 ? u ^ (r & 15) : u));
        }
    };
    // the outputs the reverse pass adds into, with two slices: slice 0 dq,
    // slice 1 dk, slice 0 the token arrays
    auto zero_outputs = [&](int c0) {
        float* dst = (sl == 0 ? J.dq : J.dk_out) + (tok0 + c0) * DK;
        const int n4 = min(kC, T - c0) * DK / 4;
        for (int x = lane; x < n4; x += 64) reinterpret_cast<f32x4*>(dst)[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sl == 0 && lane < kC && c0 + lane < T) {
            J.dalpha[tok0 + c0 + lane] = 0.f;
            if (J.dbeta) J.dbeta[tok0 + c0 + lane] = 0.f;
            if (J.dbeta_w) J.dbeta_w[tok0 + c0 + lane] = 0.f;
        }
    };

    // Prologue: S0; k, v and gates of the first chunks; T(0) and B(1).
    for (int x = tid; x < kSL * DK; x += NTH) Ss[x / DK * L1 + x % DK] = J.S0 ? J.S0[s_base + x] : 0.f;
    if constexpr (GDN)
        for (int x = tid; x < 2 * kC * LT; x += NTH) Tm[x / (kC * LT)][x % (kC * LT)] = 0.f;  // T's upper right block stays zero
    if (w == 3) {
        fetch_k(0);
        if (VW == 3) fetch_v(0);
        put_k(0);
        if (VW == 3) put_v(0);
        if constexpr (GDN) {
            if (NC > 1) {
                fetch_k(1);
                put_k(1);
            }
            fetch_k(2);
        } else {
            fetch_k(1);
        }
        if (VW == 3) fetch_v(1);
    } else if (w == VW) {  // (the delta rule's put_v needs no gates)
        fetch_v(0);
        put_v(0);
        fetch_v(1);
    }
    __syncthreads();
    if constexpr (GDN) {
        if (w == 0) {
            k_gram(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            solve_unit_lower<LB, LT>(Bm[0], gt[0].bet, Tm[0], lane);
        } else if (w == 3 && NC > 1) {
            k_gram(1);
        }
    }
    __syncthreads();
    // Each wave runs its own copy of the loop (W a constant), so the registers
    // wave 3 fetches into are never merged with other waves' values, which
    // would make the compiler wait for the loads where they are issued.
    auto run = [&](auto wc) {
        constexpr int W = decltype(wc)::value;
        constexpr int MS = kSL * DK / 4 / 64;  // 16-byte pieces of the state per lane
        // The state's tiles stay in the registers of the wave that updates them
        // (tile W + NW it: value rows 32 (tile / NJ) .., key columns 32 (tile % NJ) ..);
        // Ss holds a copy for the X products.
        constexpr int NT = (2 * NJ - W + NW - 1) / NW;
        f32x16 st[NT > 0 ? NT : 1];
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            const int tile = W + NW * it, I = tile / NJ, Jt = tile - I * NJ;
#pragma unroll
            for (int e = 0; e < 16; ++e) st[it][e] = Ss[(32 * I + row(e)) * L1 + 32 * Jt + l32];
        }
        __syncthreads();

        for (int n = 0; n < NC; ++n) {
            const int c0 = n * kC;
            const float* Kn = Ks[n % NB];
            const ChunkGatesLds& gn = gt[n % NB];
            float* Un = Us[n & 1];
            if constexpr (GDN) {
                if constexpr (W == 1 || W == 2) {  // X = beta V - beta gamma K S^T, value columns 32 (W - 1) ..
                    constexpr int I = W - 1;
                    // (K S^T with k exact in bf16; the row scalings after the product)
                    const f32x16 c = chain8_t<SPLIT, DK / 16, true>(
                        [&](int i) { return lds_f32x8(&Kn[l32 * L1 + 16 * i + 8 * kg]); },
                        [&](int i) { return lds_f32x8(&Ss[(32 * I + l32) * L1 + 16 * i + 8 * kg]); }, f32x16{});
                    const f32x16 bw16 = acc_rows16(gn.bw, kg), bg16 = acc_rows16(gn.bg, kg);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int t = row(e), y = t * LU + 32 * I + l32;
                        Un[y] = bw16[e] * Un[y] - bg16[e] * c[e];
                    }
                } else if constexpr (W == 0) {
                    if (n + 1 < NC) solve_unit_lower<LB, LT>(Bm[(n + 1) & 1], gt[(n + 1) % NB].bet, Tm[(n + 1) & 1], lane);
                    if (NW == 4 && slices == 2) zero_outputs(c0);
                } else if constexpr (W >= 4) {  // eight waves: a quarter of the state's store each, beside X
                    stash(n, std::integral_constant<int, MS * (W - 4) / 4>{}, std::integral_constant<int, MS * (W - 3) / 4>{});
                } else if constexpr (W == 3) {
                    if (n + 2 < NC) put_k(n + 2);
                    fetch_k(n + 3 < NC ? n + 3 : NC - 1);
                }
                __syncthreads();
                if constexpr (W == 1 || W == 2) {  // diag(e^{g_C - g}) U, U = T X in place, on this wave's X columns
                    constexpr int I = W - 1;
                    const float* Tn = Tm[n & 1];
                    const f32x16 c = chain8_t<SPLIT, kC / 16>(
                        [&](int i) { return lds_f32x8(&Tn[l32 * LT + 16 * i + 8 * kg]); },
                        [&](int i) { return lds_col8<LU>(&Un[(16 * i + 8 * kg) * LU + 32 * I + l32]); }, f32x16{});
                    const f32x16 dd16 = acc_rows16(gn.Dd, kg);
#pragma unroll
                    for (int e = 0; e < 16; ++e) Un[row(e) * LU + 32 * I + l32] = dd16[e] * c[e];
                    // four waves: a quarter of the state's store each
                    if constexpr (NW == 4)
                        stash(n, std::integral_constant<int, MS * (W + 1) / 4>{}, std::integral_constant<int, MS * (W + 2) / 4>{});
                } else if constexpr (W == 3) {
                    if (n + 2 < NC) k_gram(n + 2);
                }
                if constexpr (W == VW) {  // v of the next chunk into its U buffer, which no wave reads before the next X
                    if (n + 1 < NC) put_v(n + 1);
                    fetch_v(n + 2 < NC ? n + 2 : NC - 1);
                }
                if constexpr (W == 4) {
                    if (slices == 2) zero_outputs(c0);
                } else if constexpr (NW == 4 && W == 0) {  // four waves, wave 0: the first half of the state's store
                    stash(n, std::integral_constant<int, 0>{}, std::integral_constant<int, MS / 2>{});
                }
                __syncthreads();
            } else {
                if constexpr (W == 3) {
                    if (n + 1 < NC) {
                        put_k(n + 1);
                        put_v(n + 1);
                    }
                    fetch_k(n + 2 < NC ? n + 2 : NC - 1);
                    fetch_v(n + 2 < NC ? n + 2 : NC - 1);
                    if (NW == 4 && slices == 2) zero_outputs(c0);
                } else if constexpr (W == 0) {
                    if (NW == 8 && slices == 2) zero_outputs(c0);
                    if constexpr (NW == 4) stash(n, std::integral_constant<int, 0>{}, std::integral_constant<int, MS>{});
                } else if constexpr (W >= 4) {  // a quarter of the state's store each
                    stash(n, std::integral_constant<int, MS * (W - 4) / 4>{}, std::integral_constant<int, MS * (W - 3) / 4>{});
                }
                __syncthreads();  // the stash reads Ss before the update rewrites it
            }
            // S <- gamma_C S + U^T diag(e^{g_C - g}) K
#pragma unroll
            for (int it = 0; it < NT; ++it) {
                const int tile = W + NW * it, I = tile / NJ, Jt = tile - I * NJ;
                f32x16 c = gn.gC[0] * st[it];
                c = chain8_t<SPLIT, kC / 16, false, true>(
                    [&](int i) { return lds_col8<LU>(&Un[(16 * i + 8 * kg) * LU + 32 * I + l32]); },
                    [&](int i) { return lds_col8<L1>(&Kn[(16 * i + 8 * kg) * L1 + 32 * Jt + l32]); }, c);
                st[it] = c;
#pragma unroll
                for (int e = 0; e < 16; ++e) Ss[(32 * I + row(e)) * L1 + 32 * Jt + l32] = c[e];
            }
            __syncthreads();
        }
    };
    if (w == 0) run(std::integral_constant<int, 0>{});
    else if (w == 1) run(std::integral_constant<int, 1>{});
    else if (w == 2) run(std::integral_constant<int, 2>{});
    else if (w == 3) run(std::integral_constant<int, 3>{});
    else if constexpr (NW == 8) {
        if (w == 4) run(std::integral_constant<int, 4>{});
        else if (w == 5) run(std::integral_constant<int, 5>{});
        else if (w == 6) run(std::integral_constant<int, 6>{});
        else run(std::integral_constant<int, 7>{});
    }
}

// ---------------------------------------------------------------------------
// The reverse chunk pass.
template <int MODE, int DK, typename E>
__global__ __launch_bounds__(kThreadsR) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_chunk_kernel(
    BwdJob J) {
    constexpr bool GDN = MODE == 0;
    // bf16 data: the products in split bf16 (about 16 significant bits each)
    constexpr bool SPLIT = std::is_same<E, uint16_t>::value;
    // key-column tiles: wave 4 + j (j < NJ) owns dq tile j, wave j owns dk tile j
    constexpr int NJ = DK / 32;
    // Rows of the key-wide arrays and of the 32x32 matrices are 16-byte rows
    // (operands along a row come in 16-byte reads; down a column, the rows
    // r and r + 8 of the two lane halves land 32 banks apart).
    constexpr int L1 = DK + 4;
    constexpr int LP = kC + 4;
    __shared__ __align__(16) float Qs[kC * L1];
    __shared__ __align__(16) float Ks[kC * L1];
    // state entering the chunk: with rows of 64 floats or more, unpadded with
    // the 16-byte units of row r XOR-permuted by r mod 16 (as the states pass
    // stores it), so it arrives by LDS-direct loads of 1 KB; else padded rows
    constexpr bool SWZ = DK >= 64;
    __shared__ __align__(16) float Ss[kSL * (SWZ ? DK : L1)];
    __shared__ __align__(16) float dSs[kSL * L1];  // gradient at the state leaving it, then entering it
    __shared__ float Vs[kC * LV];    // V, then dX
    __shared__ float dOs[kC * LV];
    __shared__ float Us[kC * LV];    // V, then X, then U
    __shared__ float dUs[kC * LV];
    __shared__ __align__(16) float Bm[GDN ? kC * LB : 4];
    __shared__ __align__(16) float Pm[kC * LP];
    __shared__ __align__(16) float Tm[GDN ? kC * LP : 1];
    __shared__ __align__(16) float dQKm[kC * LP];  // dP o Gamma
    __shared__ __align__(16) float dKKm[GDN ? kC * LP : 1];
    __shared__ __align__(16) float G2[kC];
    __shared__ __align__(16) float bet[kC];
    __shared__ __align__(16) float gam[kC];
    __shared__ __align__(16) float Dd[kC];
    __shared__ __align__(16) float bw[kC];
    __shared__ __align__(16) float bg[kC];
    __shared__ float gC[1];
    __shared__ float dgp[16 * kC];   // per-product contributions to dg (fixed slots)
    __shared__ float dbp[8 * kC];    // ... to dbeta
    __shared__ float dgc[16];        // ... to dg_C

    const int slices = J.dv / kSL;
    int bh, slice;
    unit_part(blockIdx.x, J.BH, slices, bh, slice);  // a head's slices share its input reads in L2
    const int r0 = slice * kSL;
    int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int l32 = lane & 31, kg = lane >> 5;
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
    // index of S[r][c] in Ss
    auto sx = [&](int r, int c) { return SWZ ? r * DK + 4 * ((c >> 2) ^ (r & 15)) + (c & 3) : r * L1 + c; };
    // eight rows r0 .. r0 + 7 of S's column c
    auto s_col8 = [&](int r0, int c) {
        f32x8 x;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = Ss[sx(r0 + j, c)];
        return x;
    };
    // S[r][c .. c + 7] (c a multiple of 8)
    auto s_row8 = [&](int r, int c) {
        if constexpr (SWZ) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(&Ss[sx(r, c)]);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(&Ss[sx(r, c + 4)]);
            return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
            return lds_f32x8(&Ss[r * L1 + c]);
        }
    };
    // a group's eight operands (k = 16 i + 8 kg + j): along a 16-byte row, along
    // a row of a value-wide array (stride LV, not 16-byte), down a column
    auto rowv8 = [](const float* p) {
        f32x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = p[j];
        return r;
    };
    int k8 = 8 * kg;
    // a sum over value rows into its output: stored (one slice) or added onto
    // the zeros the states pass wrote (two slices)
    auto put = [&](float* p, float x) {
        if (slices == 1)
            *p = x;
        else
            unsafeAtomicAdd(p, x);
    };

    for (int x = tid; x < kSL * DK; x += kThreadsR) dSs[x / DK * L1 + x % DK] = J.dST ? J.dST[s_base + x] : 0.f;
    if constexpr (GDN)
        for (int x = tid; x < kC * LP; x += kThreadsR) Tm[x] = 0.f;  // T's upper right block stays zero

    // The next chunk's (in reverse order) q, k, v, dO and gates are fetched
    // into registers during this one's last two phases (unconditional loads
    // from a clamped token index; masking on the way into LDS).  Issued
    // earlier, the registers would be live through the phases with the most
    // accumulators.
    // (16-byte loads: EV elements each; RK, RV loads per row)
    constexpr int EV = 16 / (int)sizeof(E), RK = DK / EV, RV = kSL / EV;
    constexpr int QL = kC * RK, VL = kC * RV;  // loads per chunk
    constexpr int NK = (QL + kThreadsR - 1) / kThreadsR, NV = (VL + kThreadsR - 1) / kThreadsR;
    uint4 pq[NK], pk[NK], pv[NV], pd[NV];
    float pa = 1.f, pb = 0.f, pw = 0.f;
    auto fetch = [&](int n) {
        const int cn = n * kC;
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int x = min(tid + m * kThreadsR, QL - 1), t = min(cn + x / RK, T - 1);
            const size_t gi = (tok0 + t) * DK + (x % RK) * EV;
            pq[m] = *reinterpret_cast<const uint4*>(q + gi);
            pk[m] = *reinterpret_cast<const uint4*>(k + gi);
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = min(tid + m * kThreadsR, VL - 1), t = min(cn + x / RV, T - 1);
            const size_t gi = (tok0 + t) * dv + r0 + (x % RV) * EV;
            pv[m] = *reinterpret_cast<const uint4*>(v + gi);
            pd[m] = dO ? *reinterpret_cast<const uint4*>(dO + gi) : uint4{0u, 0u, 0u, 0u};
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
    // The stored state entering chunk n goes into Ss: for the first chunk
    // here, for each later one during the previous chunk's last phase, which
    // no longer reads Ss.  With rows of 64 floats or more, LDS-direct loads
    // (a wave's 16-byte load puts 1 KB into LDS, no registers: the stored
    // layout is Ss's); they are complete once vmcnt is 0, which the loop waits
    // for before the barrier that starts a chunk.  Rows of 32: 16-byte loads
    // and writes at the chunk's start.
    auto load_state = [&](int cn) {
        const float* src = J.ckpt + (((size_t)bh * J.nchunks + cn) * dv + r0) * DK;
        if constexpr (SWZ) {
#pragma unroll
            for (int b = w; b < kSL * DK / 256; b += kThreadsR / 64)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 256 * b + 4 * lane),
                                                 (__attribute__((address_space(3))) void*)(Ss + 256 * b), 16, 0, 0);
        } else {
            constexpr int NS4 = kSL * DK / 4 / kThreadsR;
            float4 sv[NS4];
#pragma unroll
            for (int m = 0; m < NS4; ++m) sv[m] = reinterpret_cast<const float4*>(src)[tid + m * kThreadsR];
#pragma unroll
            for (int m = 0; m < NS4; ++m) {
                const int x = 4 * (tid + m * kThreadsR);
                *reinterpret_cast<float4*>(Ss + x / DK * L1 + x % DK) = sv[m];
            }
        }
    };
    load_state(J.nchunks - 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    for (int n = J.nchunks - 1; n >= 0; --n) {
        // The lane indices are opaque to the compiler from here on, so the
        // address arithmetic built on them is redone in the loop rather than
        // hoisted out of it into hundreds of live registers.
        asm volatile("" : "+v"(tid), "+v"(lane), "+v"(l32), "+v"(kg), "+v"(k8));
        const int c0 = n * kC;
        __syncthreads();  // the previous chunk is done with every array
        if (!SWZ && n < J.nchunks - 1) load_state(n);
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int x = tid + m * kThreadsR, t = x / RK, y = t * L1 + (x % RK) * EV;
            if (QL % kThreadsR == 0 || x < QL) {
                const bool in = c0 + t < T;
                float fq[EV], fk[EV];
                unpack16(pq[m], fq);
                unpack16(pk[m], fk);
#pragma unroll
                for (int i = 0; i < EV; i += 4) {
                    *reinterpret_cast<f32x4*>(&Qs[y + i]) =
                        in ? f32x4{fq[i], fq[i + 1], fq[i + 2], fq[i + 3]} : f32x4{0.f, 0.f, 0.f, 0.f};
                    *reinterpret_cast<f32x4*>(&Ks[y + i]) =
                        in ? f32x4{fk[i], fk[i + 1], fk[i + 2], fk[i + 3]} : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int x = tid + m * kThreadsR, t = x / RV, y = t * LV + (x % RV) * EV;
            if (VL % kThreadsR == 0 || x < VL) {
                const bool in = c0 + t < T;
                float fv[EV], fd[EV];
                unpack16(pv[m], fv);
                unpack16(pd[m], fd);
#pragma unroll
                for (int i = 0; i < EV; ++i) {
                    const float vv = in ? fv[i] : 0.f;
                    Vs[y + i] = vv;
                    Us[y + i] = vv;
                    dOs[y + i] = in ? fd[i] : 0.f;
                }
            }
        }
        for (int x = tid; x < 16 * kC; x += kThreadsR) dgp[x] = 0.f;
        for (int x = tid; x < 8 * kC; x += kThreadsR) dbp[x] = 0.f;
        if (tid < 16) dgc[tid] = 0.f;
        if (w == 0) chunk_gates<GDN>(pa, pb, pw, c0, T, lane, G2, gam, Dd, bet, bw, bg, gC);
        __syncthreads();

        // Roles (8 waves): dq owners 4 + j and dk owners j (j < NJ) keep their
        // tiles in registers for the whole chunk; the rest of the work is
        // spread per phase below.
        const bool qown = w >= 4 && w - 4 < NJ, kown = w < NJ;
        const int jq = w - 4, jk = w;  // the owned tiles
        f32x16 acc = {};   // dq tile jq (qown) or dk tile jk (kown)
        f32x16 ksT = {};   // waves 2, 3 (delta rule): (K S^T)^T on value columns 32 (w - 2) .., kept to phase 5
        // dS tiles, from phase 2 to phase 5: wave 7 two (6, 7), waves 4, 2, 5, 3
        // one each (0, 1, 2, 3), waves 0, 1 one each (4, 5); wave 6 forms dA in
        // phase 5 instead
        f32x16 dsc[2];
        float dss[2] = {0.f, 0.f};
        auto ds_tile = [&](int h) {
            if (w == 7) return 6 + h;
            if (h == 1) return 2 * NJ;
            return w == 4 ? 0 : w == 2 ? 1 : w == 5 ? 2 : w == 3 ? 3 : w < 2 ? 4 + w : 2 * NJ;
        };
        const bool ds_wave = w != 6;
        constexpr int G1 = kC / 16;
        // Phase 1: B and then T (wave 0, delta rule), P (wave 1), X (waves 2, 3,
        // delta rule) or dU = Kd dS'^T (waves 2, 3, linear attention), and the dq
        // owners' dQ = diag(gamma) dO S (+ its dg share)
        if (GDN && w == 0) {
            auto kr = [&](int i) { return lds_f32x8(&Ks[l32 * L1 + 16 * i + k8]); };
            const f32x16 c = chain8_t<SPLIT, DK / 16, true, true>(kr, kr, f32x16{});
            const f32x16 g16 = acc_rows16(G2, kg); const float gs = G2[l32];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                Bm[t * LB + l32] = l32 < t ? __builtin_amdgcn_exp2f(g16[e] - gs) * c[e] : 0.f;
            }
            // the same wave solves right away: its own B rows are complete once
            // its LDS writes are
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            solve_unit_lower<LB, LP>(Bm, bet, Tm, lane);
        } else if (w == 1) {
            const f32x16 c = chain8_t<SPLIT, DK / 16, true, true>(
                [&](int i) { return lds_f32x8(&Qs[l32 * L1 + 16 * i + k8]); },
                [&](int i) { return lds_f32x8(&Ks[l32 * L1 + 16 * i + k8]); }, f32x16{});
            const f32x16 g16 = acc_rows16(G2, kg); const float gs = G2[l32];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                Pm[t * LP + l32] = l32 <= t ? __builtin_amdgcn_exp2f(g16[e] - gs) * c[e] : 0.f;
            }
        } else if (GDN && (w == 2 || w == 3)) {
            const int I = w - 2;
            // (K S^T)^T = S K^T with the token along the lanes: X_t = beta_t V_t - beta_t gamma_t (K S^T)_t
            // is written row by row, and the tile serves <dX_t, (K S^T)_t> in phase 5 as an in-lane sum
            ksT = chain8_t<SPLIT, DK / 16, false, true>(
                [&](int i) { return s_row8(32 * I + l32, 16 * i + k8); },
                [&](int i) { return lds_f32x8(&Ks[l32 * L1 + 16 * i + k8]); }, f32x16{});
            const float b = bw[l32], nbg = -bg[l32];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int y = l32 * LV + 32 * I + row(e);
                Us[y] = b * Us[y] + nbg * ksT[e];
            }
        } else if (!GDN && (w == 2 || w == 3)) {  // GLA: dU = Kd dS'^T
            const int I = w - 2;
            const f32x16 c = chain8_t<SPLIT, DK / 16, true>(
                [&](int i) { return lds_f32x8(&Ks[l32 * L1 + 16 * i + k8]); },
                [&](int i) { return lds_f32x8(&dSs[(32 * I + l32) * L1 + 16 * i + k8]); }, f32x16{});
            const f32x16 dd16 = acc_rows16(Dd, kg);
#pragma unroll
            for (int e = 0; e < 16; ++e) dUs[row(e) * LV + 32 * I + l32] = dd16[e] * c[e];
        } else if (qown) {
            // dO exact in bf16, gamma applied to the rows after
            acc = chain8_t<SPLIT, kSL / 16, true>([&](int i) { return rowv8(&dOs[l32 * LV + 16 * i + k8]); },
                                         [&](int i) { return s_col8(16 * i + k8, 32 * jq + l32); }, acc);
            const f32x16 gam16 = acc_rows16(gam, kg);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] *= gam16[e];
            f32x16 x;
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = acc[e] * Qs[row(e) * L1 + 32 * jq + l32];
            store_row_sums(x, dgp + jq * kC, l32, kg, 1.f);  // dg slots 0..3
        }
        __syncthreads();
        // Phase 2: U = T X (waves 2, 3) and dU = Kd dS'^T (waves 0, 1) with the
        // delta rule; the first part of the dS tiles, gamma_C dS' + dO^T diag(gamma) Q,
        // and <dS', S> (the dS waves, held in registers until phase 5: dS' is read
        // until then)
        if (GDN && (w == 2 || w == 3)) {
            const int I = w - 2;
            const f32x16 c = chain8_t<SPLIT, kC / 16>(
                [&](int i) { return lds_f32x8(&Tm[l32 * LP + 16 * i + k8]); },
                [&](int i) { return lds_col8<LV>(&Us[(16 * i + k8) * LV + 32 * I + l32]); }, f32x16{});
#pragma unroll
            for (int e = 0; e < 16; ++e) Us[row(e) * LV + 32 * I + l32] = c[e];
        } else if (GDN && w < 2) {
            const int I = w;
            const f32x16 c = chain8_t<SPLIT, DK / 16, true>(
                [&](int i) { return lds_f32x8(&Ks[l32 * L1 + 16 * i + k8]); },
                [&](int i) { return lds_f32x8(&dSs[(32 * I + l32) * L1 + 16 * i + k8]); }, f32x16{});
            const f32x16 dd16 = acc_rows16(Dd, kg);
#pragma unroll
            for (int e = 0; e < 16; ++e) dUs[row(e) * LV + 32 * I + l32] = dd16[e] * c[e];
        }
        if (ds_wave) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tile = ds_tile(h);
                if (tile < 2 * NJ) {
                    const int I = tile / NJ, Jt = tile - I * NJ;
                    f32x16 c;
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float d = dSs[(32 * I + row(e)) * L1 + 32 * Jt + l32];
                        ss += d * Ss[sx(32 * I + row(e), 32 * Jt + l32)];
                        c[e] = gC[0] * d;
                    }
                    // dO gamma on the dO side, so q stays exact in bf16
                    dsc[h] = chain8_t<SPLIT, G1, false, true>(
                        [&](int i) {
                            const int t = 16 * i + k8;
                            f32x8 r = lds_col8<LV>(&dOs[t * LV + 32 * I + l32]);
#pragma unroll
                            for (int j = 0; j < 8; ++j) r[j] *= gam[t + j];
                            return r;
                        },
                        [&](int i) { return lds_col8<L1>(&Qs[(16 * i + k8) * L1 + 32 * Jt + l32]); }, c);
                    dss[h] = ss;
                }
            }
        }
        __syncthreads();
        // Phase 3: dP (waves 4 and 5 both form it: wave 4 writes dP * Gamma, wave 5
        // the row and column sums of dP * P), dU += P^T dO (waves 0, 1 with the
        // delta rule, 2, 3 without), the dk owners' dK += Kd-part
        if (w == 4 || w == 5) {
            const f32x16 c = chain8_t<SPLIT, kSL / 16, true>([&](int i) { return rowv8(&dOs[l32 * LV + 16 * i + k8]); },
                                                    [&](int i) { return rowv8(&Us[l32 * LV + 16 * i + k8]); },
                                                    f32x16{});
            if (w == 4) {
                const f32x16 g16 = acc_rows16(G2, kg); const float gs = G2[l32];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = row(e);
                    dQKm[t * LP + l32] = l32 <= t ? c[e] * __builtin_amdgcn_exp2f(g16[e] - gs) : 0.f;
                }
            } else {
                f32x16 L;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = row(e);
                    L[e] = l32 <= t ? c[e] * Pm[t * LP + l32] : 0.f;
                }
                store_row_sums(L, dgp + 8 * kC, l32, kg, 1.f);   // dg slot 8
                store_col_sums(L, dgp + 9 * kC, l32, kg, -1.f);  // dg slot 9
            }
        }
        if (GDN ? w < 2 : (w == 2 || w == 3)) {
            const int I = GDN ? w : w - 2;
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
            c = chain8_t<SPLIT, kC / 16, false, true>([&](int i) { return lds_col8<LP>(&Pm[(16 * i + k8) * LP + l32]); },
                                             [&](int i) { return lds_col8<LV>(&dOs[(16 * i + k8) * LV + 32 * I + l32]); },
                                             c);
#pragma unroll
            for (int e = 0; e < 16; ++e) dUs[row(e) * LV + 32 * I + l32] = c[e];
        }
        if (kown) {  // dKd = U dS'
            const f32x16 c = chain8_t<SPLIT, kSL / 16>(
                [&](int i) { return rowv8(&Us[l32 * LV + 16 * i + k8]); },
                [&](int i) { return lds_col8<L1>(&dSs[(16 * i + k8) * L1 + 32 * jk + l32]); }, f32x16{});
            const f32x16 dd16 = acc_rows16(Dd, kg);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] += dd16[e] * c[e];
        }
        __syncthreads();
        // Phase 4: dX = T^T dU (delta rule, waves 0, 1; computed as dX^T = dU^T T, the token
        // along the lanes, so <dX_t, V_t> is an in-lane sum; dX replaces V row by row); the
        // owners' dQ, dK += dQK parts
        if (GDN && w < 2) {
            const int I = w;
            const f32x16 c = chain8_t<SPLIT, kC / 16>(
                [&](int i) { return lds_col8<LV>(&dUs[(16 * i + k8) * LV + 32 * I + l32]); },
                [&](int i) { return lds_col8<LP>(&Tm[(16 * i + k8) * LP + l32]); }, f32x16{});
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
        if (qown)
            acc = chain8_t<SPLIT, kC / 16, false, true>(
                [&](int i) { return lds_f32x8(&dQKm[l32 * LP + 16 * i + k8]); },
                [&](int i) { return lds_col8<L1>(&Ks[(16 * i + k8) * L1 + 32 * jq + l32]); }, acc);
        if (kown)
            acc = chain8_t<SPLIT, kC / 16, false, true>(
                [&](int i) { return lds_col8<LP>(&dQKm[(16 * i + k8) * LP + l32]); },
                [&](int i) { return lds_col8<L1>(&Qs[(16 * i + k8) * L1 + 32 * jk + l32]); }, acc);
        __syncthreads();
        // the next chunk's inputs are in flight through phases 5 and 6
        if (n > 0) fetch(n - 1);
        // Phase 5: dRw (dk owners), dA with dKK and its sums (wave 6), <dRw, K>
        // (waves 2, 3), the rest of the dS tiles (the dS waves)
        if constexpr (GDN) {
            if (kown) {  // dRw = -dX S
                const f32x16 c = chain8_t<SPLIT, kSL / 16>(
                    [&](int i) { return -rowv8(&Vs[l32 * LV + 16 * i + k8]); },
                    [&](int i) { return s_col8(16 * i + k8, 32 * jk + l32); }, f32x16{});
                const f32x16 bg16 = acc_rows16(bg, kg);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] += bg16[e] * c[e];
            }
            if (w == 6) {  // dA = strict_lower(-dX U^T): dKK, then the row and column sums of dA o B
                const f32x16 c = chain8_t<SPLIT, kSL / 16>([&](int i) { return -rowv8(&Vs[l32 * LV + 16 * i + k8]); },
                                                  [&](int i) { return rowv8(&Us[l32 * LV + 16 * i + k8]); },
                                                  f32x16{});
                f32x16 xb, xa;
                const float gs = G2[l32];
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {  // rows 8 b4 + 4 kg .. + 3: the gates as 16-byte reads
                    const f32x4 g = *reinterpret_cast<const f32x4*>(&G2[8 * b4 + 4 * kg]);
                    const f32x4 bt = *reinterpret_cast<const f32x4*>(&bet[8 * b4 + 4 * kg]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 4 * b4 + r, t = row(e);
                        const float da = l32 < t ? c[e] : 0.f;
                        // (a select: above the diagonal the exponent is not bounded)
                        dKKm[t * LP + l32] = l32 < t ? bt[r] * c[e] * __builtin_amdgcn_exp2f(g[r] - gs) : 0.f;
                        const float b = Bm[t * LB + l32];
                        xb[e] = da * b;
                        xa[e] = da * bt[r] * b;
                    }
                }
                store_row_sums(xb, dbp + 6 * kC, l32, kg, 1.f);    // dbeta slot 6 (dg: beta_t times it)
                store_col_sums(xa, dgp + 15 * kC, l32, kg, -1.f);  // dg slot 15
            }
            if (w == 2 || w == 3) {  // <dRw_t, K_t> = -<dX_t, (K S^T)_t> over this wave's value columns
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
        }
        // dV = diag(bw) dX (delta rule) or dU (linear attention), row-major from LDS
        for (int x = tid; x < kC * kSL; x += kThreadsR) {
            const int t = x / kSL, i = x % kSL;
            if (c0 + t < T)
                J.dv_out[(tok0 + c0 + t) * dv + r0 + i] = GDN ? bw[t] * Vs[t * LV + i] : dUs[t * LV + i];
        }
        // dS = gamma_C dS' + dO^T diag(gamma) Q - dX^T diag(beta gamma) K: the last
        // term (delta rule; k exact in bf16, beta gamma on the dX side), then dS into LDS
        if (ds_wave) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tile = ds_tile(h);
                if (tile < 2 * NJ) {
                    const int I = tile / NJ, Jt = tile - I * NJ;
                    f32x16 c = dsc[h];
                    if constexpr (GDN)
                        c = chain8_t<SPLIT, G1, false, true>(
                            [&](int i) {
                                const int t = 16 * i + k8;
                                f32x8 r;
#pragma unroll
                                for (int j = 0; j < 8; ++j) r[j] = -bg[t + j] * Vs[(t + j) * LV + 32 * I + l32];
                                return r;
                            },
                            [&](int i) { return lds_col8<L1>(&Ks[(16 * i + k8) * L1 + 32 * Jt + l32]); }, c);
#pragma unroll
                    for (int e = 0; e < 16; ++e) dSs[(32 * I + row(e)) * L1 + 32 * Jt + l32] = c[e];
                    const float ss = group_sum<64>(dss[h]);
                    if (lane == 0) dgc[4 + tile] = ss;
                }
            }
        }
        __syncthreads();
        if (SWZ && n > 0) load_state(n - 1);
        // Phase 6: dK += (dKK + dKK^T) K (dk owners); dq, dk; dg -> d ln alpha (wave 7),
        // dbeta (wave 6)
        if (GDN && kown)
            acc = chain8_t<SPLIT, kC / 16, false, true>(
                [&](int i) {
                    return lds_f32x8(&dKKm[l32 * LP + 16 * i + k8]) + lds_col8<LP>(&dKKm[(16 * i + k8) * LP + l32]);
                },
                [&](int i) { return lds_col8<L1>(&Ks[(16 * i + k8) * L1 + 32 * jk + l32]); }, acc);
        if (qown || kown) {
            const int jt = qown ? jq : jk;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = row(e);
                if (c0 + t < T) {
                    if (slices > 2) {
                        const size_t o = (part_tok + c0 + t) * DK + 32 * jt + l32;
                        (qown ? pdq : pdk)[o] = acc[e];
                    } else {
                        const size_t o = (tok0 + c0 + t) * DK + 32 * jt + l32;
                        put((qown ? J.dq : J.dk_out) + o, acc[e]);
                    }
                }
            }
        }
        if (w == 7) {
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
            if (kg == 0 && c0 + t < T) {
                if (slices > 2) pdl[part_tok + c0 + t] = dg;
                else put(J.dalpha + tok0 + c0 + t, dg);  // d ln alpha until bwd_finish_kernel
            }
        }
        if (w == 6) {
            // dbeta: slots 0, 1 belong to the write strength (they come from V), the
            // rest to the erase one
            const int t = l32;
            const float dbw = dbp[t] + dbp[kC + t];
            float dbe = 0.f;
#pragma unroll
            for (int s = 2; s < 8; ++s) dbe += dbp[s * kC + t];
            if (kg == 0 && c0 + t < T) {
                if (slices > 2) {
                    if (J.dbeta_w) {
                        pdb[part_tok + c0 + t] = dbe;
                        pdbw[part_tok + c0 + t] = dbw;
                    } else {
                        pdb[part_tok + c0 + t] = dbe + dbw;
                    }
                } else {
                    const size_t tk = tok0 + c0 + t;
                    if (J.dbeta_w) {
                        put(J.dbeta + tk, dbe);
                        put(J.dbeta_w + tk, dbw);
                    } else if (J.dbeta) {
                        put(J.dbeta + tk, dbe + dbw);
                    }
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the state's LDS-direct loads
    }
    __syncthreads();
    for (int x = tid; x < kSL * DK; x += kThreadsR) J.dS0[s_base + x] = dSs[x / DK * L1 + x % DK];
}

// Sum of the per-slice partials; dalpha = d ln alpha / alpha.  dq and dk in
// 16-byte pieces (dk is a multiple of 4), then the per-token values.
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(BwdJob J) {
    const size_t n_tok = (size_t)J.BH * J.T;
    const size_t n_el = n_tok * J.dk;
    const int slices = J.dv / kSL;
    const float* pdq = J.part;
    const float* pdk = pdq + (size_t)slices * n_el;
    const float* pdl = pdk + (size_t)slices * n_el;
    const float* pdb = pdl + (size_t)slices * n_tok;
    const float* pdbw = pdb + (size_t)slices * n_tok;
    const size_t stride = (size_t)gridDim.x * kThreads, x0 = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const size_t n4 = n_el / 4;
    const f32x4* pq4 = reinterpret_cast<const f32x4*>(pdq);
    const f32x4* pk4 = reinterpret_cast<const f32x4*>(pdk);
    for (size_t x = x0; x < n4; x += stride) {
        f32x4 a = pq4[x], b = pk4[x];
        for (int s = 1; s < slices; ++s) {
            a += pq4[s * n4 + x];
            b += pk4[s * n4 + x];
        }
        reinterpret_cast<f32x4*>(J.dq)[x] = a;
        reinterpret_cast<f32x4*>(J.dk_out)[x] = b;
    }
    for (size_t tk = x0; tk < n_tok; tk += stride) {
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

// dalpha = d ln alpha / alpha (one or two value slices: the sums are in place).
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(BwdJob J) {
    const size_t n_tok = (size_t)J.BH * J.T;
    for (size_t tk = (size_t)blockIdx.x * kThreads + threadIdx.x; tk < n_tok; tk += (size_t)gridDim.x * kThreads)
        J.dalpha[tk] /= J.alpha[tk];
}

template <int MODE, int DK, typename E>
hipError_t launch_typed(const BwdJob& J, hipStream_t s) {
    const dim3 grid((unsigned)((size_t)J.BH * (J.dv / kSL)));
    hipLaunchKernelGGL((bwd_states_kernel<MODE, DK, E>), grid, dim3(64 * states_waves<E>()), 0, s, J);
    hipLaunchKernelGGL((bwd_chunk_kernel<MODE, DK, E>), grid, dim3(kThreadsR), 0, s, J);
    if (J.dv / kSL > 2) {
        const size_t n4 = (size_t)J.BH * J.T * J.dk / 4;
        const size_t want = (n4 + kThreads - 1) / kThreads;
        const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3(blocks), dim3(kThreads), 0, s, J);
    } else {
        const size_t want = ((size_t)J.BH * J.T + kThreads - 1) / kThreads;
        const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
        hipLaunchKernelGGL(bwd_finish_kernel, dim3(blocks), dim3(kThreads), 0, s, J);
    }
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
    // per-slice partials only with more than two value slices
    return (size_t)BH * nchunks * dv * dk + (slices > 2 ? slices * BH * T * (2 * (size_t)dk + 3) : 0);
}

hipError_t launch_scan_bwd(int mode, int dtype, BwdJob J, hipStream_t s) {
    J.nchunks = (J.T + kC - 1) / kC;
    J.part = J.ckpt + (size_t)J.BH * J.nchunks * J.dv * J.dk;
    if (dtype == 0)
        return mode == 0 ? launch_mode<0, float>(J, s) : launch_mode<1, float>(J, s);
    return mode == 0 ? launch_mode<0, uint16_t>(J, s) : launch_mode<1, uint16_t>(J, s);
}

}  // namespace gds
