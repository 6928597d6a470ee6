// chunk_bf16.hip -- fused bfloat16 MFMA chunk kernel (dk = dv = 128, C = 64).
//
// What it computes: the chunkwise form of the affine scan S_t = S_{t-1} E_t + f_t
// (gated delta rule: E_t = alpha_t (I - beta_t k_t k_t^T), f_t = beta_t v_t k_t^T;
// gated linear attention: E_t = alpha_t I, f_t = v_t k_t^T), o_t = S_t q_t.
// The sequence is cut into chunks; each chunk is encoded independently of the
// state, chunk states are carried in order and every chunk is read out from its
// exclusive prefix state ("Sequential Parallel Duality in Prefix Scannable
// Models", papernotes.org notes: overall framework and key design 2).  Per
// chunk of C = 64 tokens (rows; g = in-chunk cumulative log decay, gamma = e^g,
// Gamma_ts = e^(g_t - g_s) for t >= s, dec_t = e^(g_C - g_t)), with S the state
// entering the chunk:
//
//   A    = strict_lower(diag(beta) (Gamma * K K^T))        k-Gram      (MFMA)
//   T    = (I + A)^-1                                       UT solve    (fp32)
//   W    = T diag(beta gamma) K,   U~ = T diag(beta) V      WY factors  (MFMA)
//   P    = (Q K^T) * Gamma * M_incl                         scores      (MFMA)
//   U    = U~ - W S^T                                       (MFMA, needs S)
//   O    = diag(gamma) Q S^T + P U                          (MFMA, needs S)
//   S   <- gamma_C S + U^T diag(dec) K                      (MFMA, fp32 state)
//
// gated linear attention: U = V and A, T, W vanish.
//
// Mapping onto gfx950.  One workgroup of 4 waves owns one head and a 64-row
// slice of its value channels, so B*H*2 workgroups run; both slices of a head
// go to the same XCD (blocks are dealt round-robin over the 8 XCDs) so the
// second read of q and k hits that XCD's L2.  The workgroup walks the chunks
// of its head in order.  Its state slice S^T (128 keys x 64 values, fp32) never
// leaves VGPRs: wave w keeps the 16 value columns [16w, 16w+16) as eight 16x16
// MFMA accumulator tiles.  Every product runs on v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation (operands rounded to bf16); the 16x16 diagonal blocks of
// the UT solve run in fp32 on the VALU and its off-diagonal blocks on the fp32
// MFMA (v_mfma_f32_16x16x4_f32).
//
// Operand trick: an MFMA accumulator tile holds, in lane (n, g), rows 4g..4g+3
// of column n.  Concatenating two row-adjacent accumulator tiles gives, per
// lane, eight values of column n -- exactly a B operand (or, transposed, an A
// operand) whose contraction index is the tile's row index, under the lane-local
// permutation k -> {4g..4g+3, 16+4g..16+4g+3}.  A product only needs both
// operands to use the same permutation, so S^T and U feed the next MFMAs
// straight from registers; the LDS-resident operand of such a product is read
// with two 8-byte loads in the same permuted order.
//
// Tokens past T in the last chunk are identity tokens (alpha = 1, beta = 0,
// q = k = v = 0), which leave S unchanged; their outputs are not written.
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int C = 64;      // tokens per chunk
constexpr int DK = 128;    // key channels
constexpr int DV = 128;    // value channels
constexpr int DVS = 64;    // value channels per workgroup
constexpr int NT = 256;    // threads per workgroup (4 waves)
constexpr int LQ = DK + 8;  // row stride (elements) of [token][key] bf16 tiles
constexpr int LT = C + 8;   // row stride of [*][token] bf16 tiles
constexpr int LA = C + 4;   // row stride of fp32 64x64 tiles
constexpr int LX = 16 + 4;  // row stride of fp32 16x16 scratch tiles

struct Smem {
    uint16_t Q[C * LQ];     // q, [token][key]
    uint16_t K[C * LQ];     // k, [token][key]
    uint16_t KT[DK * LT];   // k transposed, [key][token]
    uint16_t VT[DVS * LT];  // v slice transposed, [value][token]
    uint16_t P[C * LT];     // scores, [token][token]
    uint16_t W[C * LQ];     // -W, [token][key]
    uint16_t Tb[C * LT];    // T diag(beta)
    uint16_t Tbg[C * LT];   // T diag(beta gamma)
    float A[C * LA];        // strict-lower A (fp32)
    float Tm[C * LA];       // T = (I + A)^-1 (fp32, lower blocks)
    float X[2][16 * LX];    // solve scratch
    uint16_t O[C * LT];     // output tile of the slice, [token][value] (bf16)
    float g[C], gam[C], dec[C], bet[C];
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
// two 4-element halves (8-byte aligned each) -> one operand
__device__ __forceinline__ bf16x8 lds44(const uint16_t* p0, const uint16_t* p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
    bf16x8 r;
    r[0] = static_cast<__bf16>(a[0]); r[1] = static_cast<__bf16>(a[1]);
    r[2] = static_cast<__bf16>(a[2]); r[3] = static_cast<__bf16>(a[3]);
    r[4] = static_cast<__bf16>(b[0]); r[5] = static_cast<__bf16>(b[1]);
    r[6] = static_cast<__bf16>(b[2]); r[7] = static_cast<__bf16>(b[3]);
    return r;
}
__device__ __forceinline__ uint2 pack4(f32x4 a) {
    const uint32_t x0 = f32_to_bf16(a[0]), x1 = f32_to_bf16(a[1]);
    const uint32_t x2 = f32_to_bf16(a[2]), x3 = f32_to_bf16(a[3]);
    return make_uint2(x0 | (x1 << 16), x2 | (x3 << 16));
}
__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ __forceinline__ uint32_t word(const uint4& u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}
// sum over the 4 lanes of a quad (DPP quad permutes)
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
    return x;
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also waits
// for every outstanding global load and store of the wave (vmcnt), which would
// stall on the next chunk's prefetch and on the o stores at every barrier.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Registers holding the next chunk while the current one is computed.
struct Prefetch {
    uint4 q[4], k[4], v[2];
    float ab;  // alpha (wave 0) or beta (wave 1) of token lane
};

template <int MODE>
__device__ __forceinline__ void load_chunk(Prefetch& p, int n, int T, size_t qk_base, size_t v_base,
                                           size_t a_base, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ alpha,
                                           const float* __restrict__ beta, int tid, bool vzero) {
    const int c0 = n * C;
    const int jc = tid & 15, tg = tid >> 4;  // q/k: rows 4tg..4tg+3, keys 8jc..8jc+7
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int tok = c0 + 4 * tg + m;
        const size_t off = qk_base + (size_t)tok * DK + 8 * jc;
        p.q[m] = tok < T ? *reinterpret_cast<const uint4*>(q + off) : make_uint4(0, 0, 0, 0);
        p.k[m] = tok < T ? *reinterpret_cast<const uint4*>(k + off) : make_uint4(0, 0, 0, 0);
    }
    const int vc = tid & 7, vt = tid >> 3;  // v: rows 2vt, 2vt+1, values 8vc..8vc+7
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int tok = c0 + 2 * vt + m;
        p.v[m] = tok < T && !vzero
                     ? *reinterpret_cast<const uint4*>(v + v_base + (size_t)tok * DV + 8 * vc)
                     : make_uint4(0, 0, 0, 0);
    }
    const int tok = c0 + (tid & 63);
    if (tid < 64) p.ab = tok < T ? alpha[a_base + tok] : 1.f;
    else if (MODE == 0 && tid < 128) p.ab = tok < T ? beta[a_base + tok] : 0.f;
}

template <int MODE>
__device__ __forceinline__ void store_chunk(Smem& sm, const Prefetch& p, int tid) {
    const int jc = tid & 15, tg = tid >> 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint4*>(&sm.Q[(4 * tg + m) * LQ + 8 * jc]) = p.q[m];
        *reinterpret_cast<uint4*>(&sm.K[(4 * tg + m) * LQ + 8 * jc]) = p.k[m];
    }
    // k transposed: element e of the thread's 8 keys, tokens 4tg..4tg+3
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        uint2 u;
        if (e & 1) {
            u.x = hi16x2(word(p.k[0], wi), word(p.k[1], wi));
            u.y = hi16x2(word(p.k[2], wi), word(p.k[3], wi));
        } else {
            u.x = lo16x2(word(p.k[0], wi), word(p.k[1], wi));
            u.y = lo16x2(word(p.k[2], wi), word(p.k[3], wi));
        }
        *reinterpret_cast<uint2*>(&sm.KT[(8 * jc + e) * LT + 4 * tg]) = u;
    }
    const int vc = tid & 7, vt = tid >> 3;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        const uint32_t u = (e & 1) ? hi16x2(word(p.v[0], wi), word(p.v[1], wi))
                                   : lo16x2(word(p.v[0], wi), word(p.v[1], wi));
        *reinterpret_cast<uint32_t*>(&sm.VT[(8 * vc + e) * LT + 2 * vt]) = u;
    }
    const int lane = tid & 63;
    if (tid < 64) {
        // in-chunk cumulative log decay: inclusive prefix sum over the wave
        float x = __logf(p.ab);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        const float last = __shfl(x, 63, 64);
        sm.g[lane] = x;
        sm.gam[lane] = __expf(x);
        sm.dec[lane] = __expf(last - x);
    } else if (MODE == 0 && tid < 128) {
        sm.bet[lane] = p.ab;
    }
}

// Lower-triangular block pairs (I >= J) of the 4x4 grid of 16x16 blocks, one
// nibble per tile: I = 0,1,1,2,2,2,3,3,3,3 and J = 0,0,1,0,1,2,0,1,2,3.
constexpr uint64_t kTileI = 0x3333222110ull;
constexpr uint64_t kTileJ = 0x3210210100ull;

// Writes the staged output tile of chunk n (64 tokens x 64 values of this
// slice) with 16-byte stores: 128 contiguous bytes per token row.
__device__ __forceinline__ void flush_o(const Smem& sm, uint16_t* __restrict__ o, size_t o_base,
                                       int n, int T, int tid) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int e = tid + m * NT;           // 512 pieces of 8 values
        const int t = e >> 3, c = (e & 7) * 8;
        if (n * C + t < T)
            *reinterpret_cast<uint4*>(o + o_base + (size_t)(n * C + t) * DV + c) =
                *reinterpret_cast<const uint4*>(&sm.O[t * LT + c]);
    }
}

// Work unit = (head, leaf): a run of consecutive chunks of one head, walked in
// order by 2 (or 4) workgroups, one per 64-row slice of the state.
//  kSequential:    one leaf per head (all chunks); S_in = S0 [heads][DV][DK] or
//                  null (zero); S_out = S_T or null; o written.
//  kLeafAggregate: 4 slices; slices 0-1 carry the value rows of f starting
//                  from 0, slices 2-3 carry the rows of E starting from the
//                  identity with v = 0, so that after the leaf S_in E + f is
//                  the leaf's action.  S_out = [units][f rows; E rows][DK].
//  kLeafOutput:    S_in = state entering each leaf [units][DV][DK]; o written;
//                  the leaf job.last_leaf writes S_T to S_out (if not null).
template <int MODE, int ROLE>
__global__ __launch_bounds__(NT, 1) void chunk_mfma_kernel(const ChunkJob job) {
    constexpr bool GDN = MODE == 0;
    constexpr int NS = ROLE == kLeafAggregate ? 4 : 2;  // 64-row slices per unit
    __shared__ Smem sm;
    const uint16_t* __restrict__ q = job.q;
    const uint16_t* __restrict__ k = job.k;
    const uint16_t* __restrict__ v = job.v;
    const float* __restrict__ alpha = job.alpha;
    const float* __restrict__ beta = job.beta;
    uint16_t* __restrict__ o = job.o;
    const int T = job.T;

    // all slices of a unit on one XCD when the grid allows it (blocks are dealt
    // round-robin over the 8 XCDs), so their repeated q/k reads share an L2
    const int units = job.heads * job.leaves;
    int u, sl;
    const int x = blockIdx.x;
    if ((units & 7) == 0) {
        const int xcd = x & 7, j = x >> 3;
        u = (j / NS) * 8 + xcd;
        sl = j % NS;
    } else {
        u = x / NS;
        sl = x % NS;
    }
    const int head = u / job.leaves, leaf = u - head * job.leaves;
    const int nb = leaf * job.leaf_chunks;
    const int ne = min(nb + job.leaf_chunks, job.nchunks);
    const bool erows = ROLE == kLeafAggregate && sl >= 2;
    const int r0 = (sl & 1) * DVS;  // first value row (or E row) of the slice
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;
    const int row = r0 + 16 * w + n16;  // state row held by this lane
    const size_t qk_base = (size_t)head * T * DK;
    const size_t v_base = (size_t)head * T * DV + r0;
    const size_t a_base = (size_t)head * T;

    // state: lane (n, g) of tile jb holds S^T[16 jb + 4g + r][16 w + n] = S[row][16jb+4g+r]
    f32x4 sacc[8];
    if (ROLE == kLeafAggregate) {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[jb][r] = erows && 16 * jb + 4 * g4 + r == row ? 1.f : 0.f;
    } else {
        const size_t sb = ((size_t)(ROLE == kSequential ? head : u) * DV + row) * DK;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
            sacc[jb] = job.S_in ? *reinterpret_cast<const f32x4*>(job.S_in + sb + 16 * jb + 4 * g4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    Prefetch pf;
    if (nb < ne)
        load_chunk<MODE>(pf, nb, T, qk_base, v_base, a_base, q, k, v, alpha, beta, tid, erows);
    for (int n = nb; n < ne; ++n) {
        lds_barrier();  // every wave is done with the previous chunk's tiles
        if (o && n > nb) flush_o(sm, o, v_base, n - 1, T, tid);
        store_chunk<MODE>(sm, pf, tid);
        if (n + 1 < ne)
            load_chunk<MODE>(pf, n + 1, T, qk_base, v_base, a_base, q, k, v, alpha, beta, tid, erows);
        // upper blocks of P inside the used contraction ranges must read as zero
        for (int e = tid; e < 2 * 16 * 16; e += NT) {
            const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int t = 32 * blk + rr, s = 32 * blk + 16 + cc;
            sm.P[t * LT + s] = 0;
        }
        lds_barrier();

        // ---- k-Gram (A) and masked decayed scores (P), lower 16x16 blocks ----
        const int njobs = GDN ? 20 : 10;
        for (int job = w; job < njobs; job += 4) {
            const bool isP = job >= (GDN ? 10 : 0);
            const int tile = isP ? job - (GDN ? 10 : 0) : job;
            const int I = (int)((kTileI >> (4 * tile)) & 15), J = (int)((kTileJ >> (4 * tile)) & 15);
            const uint16_t* left = isP ? sm.Q : sm.K;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mfma16(lds8(&left[(16 * I + n16) * LQ + 32 * kk + 8 * g4]),
                             lds8(&sm.K[(16 * J + n16) * LQ + 32 * kk + 8 * g4]), acc);
            const int s = 16 * J + n16;
            const float gs = sm.g[s];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * g4 + r;
                const float decay = __expf(sm.g[t] - gs);
                if (isP) {
                    sm.P[t * LT + s] = f32_to_bf16(t >= s ? decay * acc[r] : 0.f);
                } else {
                    sm.A[t * LA + s] = t > s ? sm.bet[t] * decay * acc[r] : 0.f;
                }
            }
        }

        if constexpr (GDN) {
            lds_barrier();
            // ---- UT solve: diagonal 16x16 blocks, wave w inverts block w ----
            {
                const int c = lane >> 2, sub = lane & 3;
                const int base = 16 * w;
                float a[16][4];
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int m = 0; m < 4; ++m) a[r][m] = sm.A[(base + r) * LA + base + 4 * m + sub];
                float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = a[r][0] * xs[0] + a[r][1] * xs[1] + a[r][2] * xs[2] + a[r][3] * xs[3];
                    p = quad_sum(p);
                    const float xr = (r == c ? 1.f : 0.f) - p;
                    if ((r & 3) == sub) xs[r >> 2] = xr;
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) sm.Tm[(base + 4 * m + sub) * LA + base + c] = xs[m];
            }
            lds_barrier();
            // ---- off-diagonal blocks: T_IJ = -T_II sum_{J<=K<I} A_IK T_KJ ----
            // product helpers (fp32 MFMA, 16x16x4): lane (n, g)
            auto mul_lds = [&](const float* X, int ldx, const float* Y, int ldy, f32x4 acc) {
                // acc += X (16x16) * Y (16x16), both in LDS; natural k mapping
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma4(X[n16 * ldx + 4 * kk + g4], Y[(4 * kk + g4) * ldy + n16], acc);
                return acc;
            };
            auto mul_acc = [&](const float* X, int ldx, f32x4 Yacc, f32x4 acc) {
                // acc += X (16x16, LDS) * Y (16x16, accumulator layout); permuted k
                const f32x4 xr = *reinterpret_cast<const f32x4*>(&X[n16 * ldx + 4 * g4]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma4(xr[kk], Yacc[kk], acc);
                return acc;
            };
            auto blkA = [&](int I, int J) { return &sm.A[16 * I * LA + 16 * J]; };
            auto blkT = [&](int I, int J) { return &sm.Tm[16 * I * LA + 16 * J]; };
            auto put = [&](float* dst, int ld, f32x4 acc, float sign) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * ld + n16] = sign * acc[r];
            };
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 keep = z;  // a wave's own X product, carried to the next stage
            if (w == 0) {         // T_10
                const f32x4 m = mul_lds(blkA(1, 0), LA, blkT(0, 0), LA, z);
                put(blkT(1, 0), LA, mul_acc(blkT(1, 1), LA, m, z), -1.f);
            } else if (w == 1) {  // T_32
                const f32x4 m = mul_lds(blkA(3, 2), LA, blkT(2, 2), LA, z);
                put(blkT(3, 2), LA, mul_acc(blkT(3, 3), LA, m, z), -1.f);
            } else if (w == 2) {  // X_21 = A_21 T_11
                keep = mul_lds(blkA(2, 1), LA, blkT(1, 1), LA, z);
                put(sm.X[0], LX, keep, 1.f);
            } else {              // X_31 = A_31 T_11
                keep = mul_lds(blkA(3, 1), LA, blkT(1, 1), LA, z);
            }
            lds_barrier();
            if (w == 0) {         // X_20 = A_20 T_00 + A_21 T_10
                keep = mul_lds(blkA(2, 1), LA, blkT(1, 0), LA, mul_lds(blkA(2, 0), LA, blkT(0, 0), LA, z));
                put(sm.X[1], LX, keep, 1.f);
            } else if (w == 1) {  // X_30 = A_30 T_00 + A_31 T_10
                keep = mul_lds(blkA(3, 1), LA, blkT(1, 0), LA, mul_lds(blkA(3, 0), LA, blkT(0, 0), LA, z));
            } else if (w == 2) {  // T_21 = -T_22 X_21
                put(blkT(2, 1), LA, mul_acc(blkT(2, 2), LA, keep, z), -1.f);
            } else {              // T_31 = -(T_32 X_21 + T_33 X_31)
                const f32x4 t = mul_lds(blkT(3, 2), LA, sm.X[0], LX, z);
                put(blkT(3, 1), LA, mul_acc(blkT(3, 3), LA, keep, t), -1.f);
            }
            lds_barrier();
            if (w == 0) {         // T_20 = -T_22 X_20
                put(blkT(2, 0), LA, mul_acc(blkT(2, 2), LA, keep, z), -1.f);
            } else if (w == 1) {  // T_30 = -(T_32 X_20 + T_33 X_30)
                const f32x4 t = mul_lds(blkT(3, 2), LA, sm.X[1], LX, z);
                put(blkT(3, 0), LA, mul_acc(blkT(3, 3), LA, keep, t), -1.f);
            }
            lds_barrier();
            // ---- bf16 right-hand-side factors: T diag(beta), T diag(beta gamma) ----
            for (int e = tid; e < C * C; e += NT) {
                const int t = e >> 6, s = e & 63;
                const float tv = s <= t ? sm.Tm[t * LA + s] : 0.f;
                const float b = sm.bet[s];
                sm.Tb[t * LT + s] = f32_to_bf16(tv * b);
                sm.Tbg[t * LT + s] = f32_to_bf16(tv * b * sm.gam[s]);
            }
            lds_barrier();
            // ---- W^T = K^T (T diag(beta gamma))^T; stored as -W [token][key] ----
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int jb = 2 * w + jj;
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        if (kk == 1 && tb < 2) continue;  // T is lower triangular
                        acc = mfma16(lds8(&sm.KT[(16 * jb + n16) * LT + 32 * kk + 8 * g4]),
                                     lds8(&sm.Tbg[(16 * tb + n16) * LT + 32 * kk + 8 * g4]), acc);
                    }
                    const f32x4 neg = {-acc[0], -acc[1], -acc[2], -acc[3]};
                    *reinterpret_cast<uint2*>(&sm.W[(16 * tb + n16) * LQ + 16 * jb + 4 * g4]) = pack4(neg);
                }
            }
        }
        lds_barrier();

        // ---- state-dependent part; wave w owns value columns [16w, 16w+16) ----
        bf16x8 sb[4];  // S^T as B operands, contraction over keys (permuted)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sb[kk] = pack8(sacc[2 * kk], sacc[2 * kk + 1]);

        f32x4 uacc[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            if constexpr (GDN) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk == 1 && tb < 2) continue;
                    acc = mfma16(lds8(&sm.Tb[(16 * tb + n16) * LT + 32 * kk + 8 * g4]),
                                 lds8(&sm.VT[(16 * w + n16) * LT + 32 * kk + 8 * g4]), acc);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint16_t* wr = &sm.W[(16 * tb + n16) * LQ + 32 * kk + 4 * g4];
                    acc = mfma16(lds44(wr, wr + 16), sb[kk], acc);
                }
                uacc[tb] = acc;
            } else {
                const uint2 u = *reinterpret_cast<const uint2*>(&sm.VT[(16 * w + n16) * LT + 16 * tb + 4 * g4]);
                uacc[tb] = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
            }
        }
        bf16x8 ub[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) ub[kk] = pack8(uacc[2 * kk], uacc[2 * kk + 1]);

        // O = diag(gamma) Q S^T + P U
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 qs = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint16_t* qr = &sm.Q[(16 * tb + n16) * LQ + 32 * kk + 4 * g4];
                qs = mfma16(lds44(qr, qr + 16), sb[kk], qs);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk == 1 && tb < 2) continue;
                const uint16_t* pr = &sm.P[(16 * tb + n16) * LT + 32 * kk + 4 * g4];
                pu = mfma16(lds44(pr, pr + 16), ub[kk], pu);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * g4 + r;
                sm.O[t * LT + 16 * w + n16] = f32_to_bf16(sm.gam[t] * qs[r] + pu[r]);
            }
        }

        // S^T <- gamma_C S^T + K^T diag(dec) U
        bf16x8 db[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f32x4 a = uacc[2 * kk], b = uacc[2 * kk + 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                a[r] *= sm.dec[32 * kk + 4 * g4 + r];
                b[r] *= sm.dec[32 * kk + 16 + 4 * g4 + r];
            }
            db[kk] = pack8(a, b);
        }
        const float gC = sm.gam[C - 1];
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
            f32x4 acc = sacc[jb] * gC;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint16_t* kr = &sm.KT[(16 * jb + n16) * LT + 32 * kk + 4 * g4];
                acc = mfma16(lds44(kr, kr + 16), db[kk], acc);
            }
            sacc[jb] = acc;
        }
    }

    if (o && ne > nb) {
        lds_barrier();
        flush_o(sm, o, v_base, ne - 1, T, tid);
    }
    float* dst = nullptr;
    if (ROLE == kSequential && job.S_out) dst = job.S_out + ((size_t)head * DV + row) * DK;
    if (ROLE == kLeafAggregate) dst = job.S_out + ((size_t)u * (DV + DK) + sl * DVS + 16 * w + n16) * DK;
    if (ROLE == kLeafOutput && job.S_out && leaf == job.last_leaf)
        dst = job.S_out + ((size_t)head * DV + row) * DK;
    if (dst) {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) *reinterpret_cast<f32x4*>(dst + 16 * jb + 4 * g4) = sacc[jb];
    }
}

}  // namespace

bool chunk_mfma_supported(int mode, int dk, int dv, int chunk) {
    (void)mode;
    return dk == DK && dv == DV && chunk == C;
}

template <int MODE>
static hipError_t launch_role(int role, const ChunkJob& job, hipStream_t stream) {
    const int units = job.heads * job.leaves;
    const dim3 block(NT);
    if (role == kSequential)
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kSequential>), dim3(2 * units), block, 0, stream, job);
    else if (role == kLeafAggregate)
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kLeafAggregate>), dim3(4 * units), block, 0, stream, job);
    else
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kLeafOutput>), dim3(2 * units), block, 0, stream, job);
    return hipGetLastError();
}

hipError_t launch_chunk_job(int mode, int role, const ChunkJob& job, hipStream_t stream) {
    return mode == 0 ? launch_role<0>(role, job, stream) : launch_role<1>(role, job, stream);
}

hipError_t launch_chunk_mfma(int mode, int BH, int T, int dk, int dv, int chunk, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta,
                             const float* S0, void* o, float* ST, hipStream_t stream) {
    (void)dk; (void)dv; (void)chunk;
    ChunkJob job{};
    job.q = static_cast<const uint16_t*>(q);
    job.k = static_cast<const uint16_t*>(k);
    job.v = static_cast<const uint16_t*>(v);
    job.alpha = alpha;
    job.beta = beta;
    job.o = static_cast<uint16_t*>(o);
    job.S_in = S0;
    job.S_out = ST;
    job.heads = BH;
    job.T = T;
    job.nchunks = (T + C - 1) / C;
    job.leaves = 1;
    job.leaf_chunks = job.nchunks;
    job.last_leaf = 0;
    return launch_chunk_job(mode, kSequential, job, stream);
}

}  // namespace gds
