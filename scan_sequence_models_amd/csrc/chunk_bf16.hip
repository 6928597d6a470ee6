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
// Mapping onto gfx950.  A workgroup of 8 waves owns one head and a 64-row slice
// of its value channels (B*H*2 workgroups on the sequential path); all slices of
// a head go to one XCD (blocks are dealt round-robin over the 8 XCDs) so their
// repeated q/k reads share that XCD's L2.  The waves specialise:
//   waves 0-1      state waves: wave w keeps the 32 value columns [32w, 32w+32)
//                  of S^T (128 keys, fp32) in four 32x32 MFMA accumulator tiles
//                  for the whole sequence and runs the S-dependent products of
//                  chunk n;
//   waves 2,3,6,7  k-Gram and scores, the off-diagonal UT-solve blocks and W
//                  for chunk n+1;
//   waves 4-5      q tile, transposed k/v tiles, the diagonal UT-solve blocks
//                  and U~ for chunk n+1.
// Chunk n+1's factors are built while chunk n's state pass runs; they meet
// through LDS (double-buffered where the phase order needs it).  All waves
// pass the same seven barriers per chunk.  Every product is
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation, bf16 operands) except the UT
// solve: its 16x16 diagonal blocks run in fp32 on the VALU and its off-diagonal
// blocks on the fp32 MFMA (16x16x4).
//
// Operand trick: a 32x32 accumulator tile holds, in lane (n, h), rows
// 8b + 4h + r (b, r < 4) of column n.  Elements 8s..8s+7 of a lane are then the
// 8 rows {16s + 8b' + 4h + r}: a B operand whose contraction index is the
// tile's row.  The state and U tiles are laid out with bits 2 and 3 of the row
// index swapped (row rho holds key/token perm5(rho)), so those 8 rows are the 8
// consecutive keys/tokens 16s + 8h .. 16s + 8h + 7, and the matching A operand
// is one natural 16-byte LDS or global read.
//
// Tokens past T in the last chunk are identity tokens (alpha = 1, beta = 0,
// q = k = v = 0), which leave S unchanged; their outputs are not written.
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int C = 64;        // tokens per chunk
constexpr int DK = 128;      // key channels
constexpr int DV = 128;      // value channels
constexpr int DVS = 64;      // value channels per workgroup
constexpr int NT = 512;      // 8 waves
constexpr int LW = DK + 8;   // row stride (elements) of -W [token][key]
constexpr int LT = C + 8;    // row stride of [*][token] bf16 tiles
constexpr int LA = C + 4;    // row stride of fp32 64x64 tiles
constexpr int LU = DVS + 4;  // row stride of U~ [token][value] (fp32)
constexpr int LX = 16 + 4;   // row stride of fp32 16x16 scratch tiles

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct Gates {
    float g[C], gam[C], dec[C], bet[C];
};

struct Smem {
    uint16_t Q[C * LW];       // q of the chunk the state waves consume next [token][key]
    uint16_t W[C * LW];       // -W of the chunk the state waves consume next
    uint16_t KT[2][DK * LT];  // k transposed [key][token] (token granules swizzled)
    uint16_t P[2][C * LT];    // scores [token][token]
    float Ut[C * LU];         // U~ [token][value]
    Gates gate[2];
    union {
        float A[C * LA];      // strict-lower A (fp32), solve phases
        struct {
            uint16_t Tb[C * LT];   // T diag(beta)
            uint16_t Tbg[C * LT];  // T diag(beta gamma)
        } t;
    } a;
    float Tm[C * LA];         // T = (I + A)^-1 (fp32, lower blocks)
    uint16_t VT[DVS * LT];    // v slice transposed [value][token] (swizzled)
    float X[2][16 * LX];      // solve scratch
    float gs[4][2][C];        // per Gram wave: g and beta of its chunk
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
template <int OFF>
__device__ __forceinline__ bf16x8 half8(const f32x16& x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[OFF + i]);
    return r;
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    const uint32_t x0 = f32_to_bf16(a), x1 = f32_to_bf16(b);
    const uint32_t x2 = f32_to_bf16(c), x3 = f32_to_bf16(d);
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
// stall on prefetches and output stores at every barrier.  The memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value,
// so that role and tile choices compile to scalar branches.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Row permutation of the state and U tiles: swap bits 2 and 3.
__device__ __forceinline__ int perm5(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// Key (state tile) or token (U / O tile) held by accumulator element e of a
// lane in half h of the wave.
__device__ __forceinline__ int elem_index(int tile, int e, int h) {
    return 32 * tile + 16 * (e >> 3) + 8 * h + 4 * ((e >> 2) & 1) + (e & 3);
}
// [row][token] tiles with 8-token granules XOR-swizzled by row, so that the
// transposed 8-byte stores spread over all LDS banks.
__device__ __forceinline__ int tsw(int row, int tok) {
    return row * LT + ((((tok >> 3) ^ (row >> 3)) & 7) << 3) + (tok & 7);
}

// Rows of chunk m of one head's [T][ld] bf16 tensor, read through a buffer
// resource whose range ends at token T: rows past the end read as zero by the
// hardware range check, with no branch.  `head` must be wave-uniform.
struct Rows {
    __amdgpu_buffer_rsrc_t r;
    int ld;
    __device__ __forceinline__ Rows(const uint16_t* head, int m, int T, int ld_) : ld(ld_) {
        // (readfirstlane: keeps the uniform size in a scalar register)
        const int valid = __builtin_amdgcn_readfirstlane(min(max(T - m * C, 0), C));
        r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(head + (size_t)m * C * ld_),
                                              (short)0, valid * ld_ * 2, 0x00020000);
    }
    // 16 bytes: columns col..col+7 of row `row` (0 <= row < C) of the chunk
    __device__ __forceinline__ uint4 at(int row, int col) const {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (row * ld + col) * 2, 0, 0));
    }
};
// Per-token float of chunk m (alpha or beta); tokens past T read as `pad`.
__device__ __forceinline__ float ldtok(const float* head, int m, int i, int T, float pad) {
    const int valid = __builtin_amdgcn_readfirstlane(min(max(T - m * C, 0), C));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(head + (size_t)m * C), (short)0, valid * 4, 0x00020000);
    const float v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
    return v + (i < valid ? 0.f : pad);  // the hardware returns 0 past the end
}
// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row broadcasts of lanes 15 and 31).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
    return x;
}

// 16x16 block products of the UT solve (fp32 MFMA, 16x16x4); lane (n16, g4).
struct Solve {
    Smem& sm;
    int n16, g4;
    // acc += X * Y, both 16x16 in LDS (natural k order)
    __device__ f32x4 mul_lds(const float* X, int ldx, const float* Y, int ldy, f32x4 acc) const {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mfma4(X[n16 * ldx + 4 * kk + g4], Y[(4 * kk + g4) * ldy + n16], acc);
        return acc;
    }
    // acc += X * Y, X in LDS, Y an accumulator tile (k = 4 g4 + kk)
    __device__ f32x4 mul_acc(const float* X, int ldx, f32x4 Yacc, f32x4 acc) const {
        const f32x4 xr = *reinterpret_cast<const f32x4*>(&X[n16 * ldx + 4 * g4]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma4(xr[kk], Yacc[kk], acc);
        return acc;
    }
    __device__ float* blkA(int I, int J) const { return &sm.a.A[16 * I * LA + 16 * J]; }
    __device__ float* blkT(int I, int J) const { return &sm.Tm[16 * I * LA + 16 * J]; }
    __device__ void put(float* dst, int ld, f32x4 acc, float sign) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * ld + n16] = sign * acc[r];
    }
};

// B operand for contraction step kk (16 rows) from accumulator tiles:
// tile kk/2, elements 8(kk%2) .. 8(kk%2)+7, rounded to bf16.
template <int N>
__device__ __forceinline__ bf16x8 sop(const f32x16 (&t)[N], int kk) {
    return (kk & 1) ? half8<8>(t[kk >> 1]) : half8<0>(t[kk >> 1]);
}

struct Unit {
    int head, leaf, sl, nb, ne, r0;
    bool erows;
};

template <int ROLE>
__device__ __forceinline__ Unit unit_of(const ChunkJob& job) {
    constexpr int NS = ROLE == kLeafAggregate ? 4 : 2;
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
    Unit un;
    un.head = u / job.leaves;
    un.leaf = u - un.head * job.leaves;
    un.sl = sl;
    un.nb = un.leaf * job.leaf_chunks;
    un.ne = min(un.nb + job.leaf_chunks, job.nchunks);
    un.erows = ROLE == kLeafAggregate && sl >= 2;
    un.r0 = (sl & 1) * DVS;
    return un;
}

// ----------------------------------------------------------------------------
// state waves (0, 1): chunk n's S-dependent products
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void state_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    const int tid = threadIdx.x, lane = tid & 63, ib = wave_id();
    const int l32 = lane & 31, h = lane >> 5;
    const int T = job.T;
    const int vcol = un.r0 + 32 * ib + l32;  // state row (value channel) of this lane

    // sacc[jt] element e = S[vcol][elem_index(jt, e, h)]
    f32x16 sacc[4];
    if (ROLE == kLeafAggregate) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[jt][e] = un.erows && elem_index(jt, e, h) == vcol ? 1.f : 0.f;
    } else {
        const int unit = ROLE == kSequential ? un.head : un.head * job.leaves + un.leaf;
        const float* src = job.S_in ? job.S_in + ((size_t)unit * DV + vcol) * DK : nullptr;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int k0 = 32 * jt + 16 * s2 + 8 * h;
                const f32x4 a = src ? *reinterpret_cast<const f32x4*>(src + k0) : f32x4{0, 0, 0, 0};
                const f32x4 b = src ? *reinterpret_cast<const f32x4*>(src + k0 + 4) : f32x4{0, 0, 0, 0};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sacc[jt][8 * s2 + r] = a[r];
                    sacc[jt][8 * s2 + 4 + r] = b[r];
                }
            }
    }

    for (int it = un.nb - 1; it < un.ne; ++it) {
        const bool act = it >= un.nb;
        const int n = it, buf = n & 1;
        const Gates& G = sm.gate[buf];
        f32x16 uacc[2];
        // ---- phase 1: U = U~ - W S^T ----
        if (act) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    uacc[tt][e] = sm.Ut[elem_index(tt, e, h) * LU + 32 * ib + l32];
                if (GDN) {
                    const uint16_t* wr = &sm.W[(32 * tt + perm5(l32)) * LW + 8 * h];
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk)
                        uacc[tt] = mfma32(lds8(wr + 16 * kk), sop(sacc, kk), uacc[tt]);
                }
            }
        }
        lds_barrier();  // 1
        // ---- phases 2-3: O = diag(gamma) Q S^T + P U for token tile tt = phase - 2, write o ----
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            if (act) {
                f32x16 acc = {};
                const uint16_t* qr = &sm.Q[(32 * tt + perm5(l32)) * LW + 8 * h];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) acc = mfma32(lds8(qr + 16 * kk), sop(sacc, kk), acc);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] *= G.gam[elem_index(tt, e, h)];
                const uint16_t* pr = &sm.P[buf][(32 * tt + perm5(l32)) * LT + 8 * h];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if (tt == 0 && ks >= 2) continue;  // P is lower triangular
                    acc = mfma32(lds8(pr + 16 * ks), sop(uacc, ks), acc);
                }
                if (job.o) {
                    uint16_t* orow = job.o + ((size_t)un.head * T + (size_t)n * C) * DV + un.r0 + 32 * ib + l32;
                    if ((n + 1) * C <= T) {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            orow[(size_t)elem_index(tt, e, h) * DV] = f32_to_bf16(acc[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int t = elem_index(tt, e, h);
                            if (n * C + t < T) orow[(size_t)t * DV] = f32_to_bf16(acc[e]);
                        }
                    }
                }
            }
            lds_barrier();  // 2, 3
        }
        // ---- phase 4: S^T <- gamma_C S^T + K^T diag(dec) U ----
        if (act) {
            bf16x8 db[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f32x16 x = uacc[ks >> 1];
                const int off = 8 * (ks & 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) x[off + i] *= G.dec[16 * ks + 8 * h + i];
                db[ks] = (ks & 1) ? half8<8>(x) : half8<0>(x);
            }
            const float gC = G.gam[C - 1];
            const uint16_t* KT = sm.KT[buf];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                f32x16 acc = sacc[jt] * gC;
                const int row = 32 * jt + perm5(l32);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma32(lds8(&KT[tsw(row, 16 * ks + 8 * h)]), db[ks], acc);
                sacc[jt] = acc;
            }
        }
        lds_barrier();  // 4
        lds_barrier();  // 5
        lds_barrier();  // 6
        lds_barrier();  // 7
    }

    float* dst = nullptr;
    if (ROLE == kSequential && job.S_out) dst = job.S_out + ((size_t)un.head * DV + vcol) * DK;
    if (ROLE == kLeafAggregate)
        dst = job.S_out + ((size_t)(un.head * job.leaves + un.leaf) * (DV + DK) + un.sl * DVS +
                           32 * ib + l32) * DK;
    if (ROLE == kLeafOutput && job.S_out && un.leaf == job.last_leaf)
        dst = job.S_out + ((size_t)un.head * DV + vcol) * DK;
    if (dst) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int k0 = 32 * jt + 16 * s2 + 8 * h;
                const f32x16& s = sacc[jt];
                *reinterpret_cast<f32x4*>(dst + k0) =
                    f32x4{s[8 * s2], s[8 * s2 + 1], s[8 * s2 + 2], s[8 * s2 + 3]};
                *reinterpret_cast<f32x4*>(dst + k0 + 4) =
                    f32x4{s[8 * s2 + 4], s[8 * s2 + 5], s[8 * s2 + 6], s[8 * s2 + 7]};
            }
    }
}

// Inverse of the unit lower-triangular 16x16 diagonal block I + A_bb, by
// forward substitution in fp32: lane (c, sub) owns column c of the inverse and
// sums the terms s = sub (mod 4) of each row; a quad reduction completes it.
__device__ __forceinline__ void diag_inverse(Smem& sm, int blk, int lane) {
    const int c = lane >> 2, sub = lane & 3;
    const int base = 16 * blk;
    float a[16][4];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) a[r][mm] = sm.a.A[(base + r) * LA + base + 4 * mm + sub];
    float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float p = a[r][0] * xs[0] + a[r][1] * xs[1] + a[r][2] * xs[2] + a[r][3] * xs[3];
        p = quad_sum(p);
        const float xr = (r == c ? 1.f : 0.f) - p;
        if ((r & 3) == sub) xs[r >> 2] = xr;
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) sm.Tm[(base + 4 * mm + sub) * LA + base + c] = xs[mm];
}

// Tb / Tbg: T diag(beta) and T diag(beta gamma) in bf16, upper part zero.
// Shared by the six prep waves (prep thread index p in 0..383).
__device__ __forceinline__ void build_tb(Smem& sm, const Gates& G, int p) {
    for (int piece = p; piece < C * C / 8; piece += 384) {
        const int t = piece >> 3, s0 = (piece & 7) * 8;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sm.Tm[t * LA + s0]);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sm.Tm[t * LA + s0 + 4]);
        float tv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tv[i] = s0 + i <= t ? x0[i] : 0.f;
            tv[4 + i] = s0 + 4 + i <= t ? x1[i] : 0.f;
        }
        uint32_t b[4], bg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = s0 + 2 * i;
            const float e0 = tv[2 * i] * G.bet[s], e1 = tv[2 * i + 1] * G.bet[s + 1];
            b[i] = f32_to_bf16(e0) | ((uint32_t)f32_to_bf16(e1) << 16);
            bg[i] = f32_to_bf16(e0 * G.gam[s]) | ((uint32_t)f32_to_bf16(e1 * G.gam[s + 1]) << 16);
        }
        *reinterpret_cast<uint4*>(&sm.a.t.Tb[t * LT + s0]) = make_uint4(b[0], b[1], b[2], b[3]);
        *reinterpret_cast<uint4*>(&sm.a.t.Tbg[t * LT + s0]) = make_uint4(bg[0], bg[1], bg[2], bg[3]);
    }
}

// ----------------------------------------------------------------------------
// k-Gram / scores / UT solve / W waves (2, 3, 6, 7): chunk n+1
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void gram_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int gi = w == 2 ? 0 : w == 3 ? 1 : w == 6 ? 2 : 3;
    const int l32 = lane & 31, h = lane >> 5;
    const int n16 = lane & 15, g4 = lane >> 4;
    const int T = job.T;
    const size_t qk_base = (size_t)un.head * T * DK;
    const size_t a_base = (size_t)un.head * T;

    // Operand rows of the wave's tiles: op0 = k rows [row0, row0+32),
    // op1 = (gi == 0 ? k : q) rows [row1, row1+32).
    //   gdn: gi 0: A00 (op0 op0), A10 (op1 op0);  gi 1: A11 (op0 op0), P11 (op1 op0);
    //        gi 2: P00 (op1 op0);  gi 3: P10 (op1 op0).   gla: gi 1..3 as gdn's P tiles.
    const uint16_t* src1 = gi == 0 ? job.k : job.q;
    const int row0 = gi == 1 ? 32 : 0, row1 = gi == 2 ? 0 : 32;
    uint4 op0[8], op1[8];
    float pa = 1.f, pb = 0.f;  // alpha and beta of token `lane`
    auto load_ops = [&](int m) {
        const Rows r0(job.k + qk_base, m, T, DK), r1(src1 + qk_base, m, T, DK);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            op0[kk] = r0.at(row0 + l32, 16 * kk + 8 * h);
            op1[kk] = r1.at(row1 + l32, 16 * kk + 8 * h);
        }
        pa = ldtok(job.alpha + a_base, m, lane, T, 1.f);
        pb = GDN ? ldtok(job.beta + a_base, m, lane, T, 0.f) : 0.f;
    };
    if (un.nb < un.ne) load_ops(un.nb);
    const Solve sv{sm, n16, g4};

    for (int it = un.nb - 1; it < un.ne; ++it) {
        const int m = it + 1;
        const bool act = m < un.ne;
        const int buf = m & 1;
        Gates& G = sm.gate[buf];
        // ---- phase 1: gates, k-Gram A and scores P of chunk m ----
        if (act) {
            const float x = wave_inclusive_sum(__logf(pa));
            float* gsl = sm.gs[gi][0];
            float* bsl = sm.gs[gi][1];
            gsl[lane] = x;
            bsl[lane] = pb;
            if (gi == 0) {
                const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
                G.g[lane] = x;
                G.gam[lane] = __expf(x);
                G.dec[lane] = __expf(last - x);
                G.bet[lane] = pb;
            }
            // tiles (isP, I, J, A operand = op1?):
            //   gdn: gi 0: A00, A10;  gi 1: A11, P11;  gi 2: P00;  gi 3: P10.
            //   gla: gi 1: P11;  gi 2: P00;  gi 3: P10.
            const int ntiles = GDN ? (gi <= 1 ? 2 : 1) : (gi == 0 ? 0 : 1);
            bool isP[2], a1[2];
            int I[2], J[2];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                if (gi == 0) { isP[ti] = false; I[ti] = ti; J[ti] = 0; a1[ti] = ti == 1; }
                else if (gi == 1) { isP[ti] = !GDN || ti == 1; I[ti] = 1; J[ti] = 1; a1[ti] = isP[ti]; }
                else if (gi == 2) { isP[ti] = true; I[ti] = 0; J[ti] = 0; a1[ti] = true; }
                else { isP[ti] = true; I[ti] = 1; J[ti] = 0; a1[ti] = true; }
            }
            // every gate value the masks need, read before any mask is written
            float grow[2][16], brow[2][16], gcol[2];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                gcol[ti] = gsl[32 * J[ti] + l32];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = 32 * I[ti] + 8 * (e >> 2) + 4 * h + (e & 3);
                    grow[ti][e] = gsl[t];
                    brow[ti][e] = bsl[t];
                }
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                if (ti >= ntiles) break;
                f32x16 acc = {};
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    acc = mfma32(as_bf16x8(a1[ti] ? op1[kk] : op0[kk]), as_bf16x8(op0[kk]), acc);
                const int s = 32 * J[ti] + l32;
                float val[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = 32 * I[ti] + 8 * (e >> 2) + 4 * h + (e & 3);
                    const float decay = __expf(grow[ti][e] - gcol[ti]);
                    val[e] = isP[ti] ? (t >= s ? decay * acc[e] : 0.f)
                                     : (t > s ? brow[ti][e] * decay * acc[e] : 0.f);
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = 32 * I[ti] + 8 * (e >> 2) + 4 * h + (e & 3);
                    if (isP[ti]) sm.P[buf][t * LT + s] = f32_to_bf16(val[e]);
                    else sm.a.A[t * LA + s] = val[e];
                }
            }
        }
        lds_barrier();  // 1
        // ---- phase 2: next chunk's operands in flight (the diagonal inverses run on waves 4-5) ----
        if (act && m + 1 < un.ne) load_ops(m + 1);
        lds_barrier();  // 2
        // ---- phases 3-5: off-diagonal blocks T_IJ = -T_II sum_K A_IK T_KJ ----
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 keep = z;
        if (GDN && act) {
            if (gi == 0) {         // T_10
                const f32x4 mm = sv.mul_lds(sv.blkA(1, 0), LA, sv.blkT(0, 0), LA, z);
                sv.put(sv.blkT(1, 0), LA, sv.mul_acc(sv.blkT(1, 1), LA, mm, z), -1.f);
            } else if (gi == 1) {  // T_32
                const f32x4 mm = sv.mul_lds(sv.blkA(3, 2), LA, sv.blkT(2, 2), LA, z);
                sv.put(sv.blkT(3, 2), LA, sv.mul_acc(sv.blkT(3, 3), LA, mm, z), -1.f);
            } else if (gi == 2) {  // X_21 = A_21 T_11
                keep = sv.mul_lds(sv.blkA(2, 1), LA, sv.blkT(1, 1), LA, z);
                sv.put(sm.X[0], LX, keep, 1.f);
            } else {               // X_31 = A_31 T_11
                keep = sv.mul_lds(sv.blkA(3, 1), LA, sv.blkT(1, 1), LA, z);
            }
        }
        lds_barrier();  // 3
        if (GDN && act) {
            if (gi == 0) {         // X_20 = A_20 T_00 + A_21 T_10
                keep = sv.mul_lds(sv.blkA(2, 1), LA, sv.blkT(1, 0), LA,
                                  sv.mul_lds(sv.blkA(2, 0), LA, sv.blkT(0, 0), LA, z));
                sv.put(sm.X[1], LX, keep, 1.f);
            } else if (gi == 1) {  // X_30 = A_30 T_00 + A_31 T_10
                keep = sv.mul_lds(sv.blkA(3, 1), LA, sv.blkT(1, 0), LA,
                                  sv.mul_lds(sv.blkA(3, 0), LA, sv.blkT(0, 0), LA, z));
            } else if (gi == 2) {  // T_21 = -T_22 X_21
                sv.put(sv.blkT(2, 1), LA, sv.mul_acc(sv.blkT(2, 2), LA, keep, z), -1.f);
            } else {               // T_31 = -(T_32 X_21 + T_33 X_31)
                const f32x4 t = sv.mul_lds(sv.blkT(3, 2), LA, sm.X[0], LX, z);
                sv.put(sv.blkT(3, 1), LA, sv.mul_acc(sv.blkT(3, 3), LA, keep, t), -1.f);
            }
        }
        lds_barrier();  // 4
        if (GDN && act) {
            if (gi == 0) {         // T_20 = -T_22 X_20
                sv.put(sv.blkT(2, 0), LA, sv.mul_acc(sv.blkT(2, 2), LA, keep, z), -1.f);
            } else if (gi == 1) {  // T_30 = -(T_32 X_20 + T_33 X_30)
                const f32x4 t = sv.mul_lds(sv.blkT(3, 2), LA, sm.X[1], LX, z);
                sv.put(sv.blkT(3, 0), LA, sv.mul_acc(sv.blkT(3, 3), LA, keep, t), -1.f);
            }
        }
        lds_barrier();  // 5
        // ---- phase 6: bf16 right-hand-side factors ----
        if (GDN && act) build_tb(sm, G, tid - 128);
        lds_barrier();  // 6
        // ---- phase 7: W^T = K^T (T diag(beta gamma))^T for key tile jt = gi; stored as -W ----
        if (GDN && act) {
            const uint16_t* KT = sm.KT[buf];
            const int jt = gi;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x16 acc = {};
                const uint16_t* tr = &sm.a.t.Tbg[(32 * tt + l32) * LT + 8 * h];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if (tt == 0 && kk >= 2) continue;  // T is lower triangular
                    acc = mfma32(lds8(&KT[tsw(32 * jt + l32, 16 * kk + 8 * h)]), lds8(tr + 16 * kk), acc);
                }
                uint16_t* wrow = &sm.W[(32 * tt + l32) * LW + 32 * jt + 4 * h];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    *reinterpret_cast<uint2*>(wrow + 8 * b) =
                        pack4(-acc[4 * b], -acc[4 * b + 1], -acc[4 * b + 2], -acc[4 * b + 3]);
            }
        }
        lds_barrier();  // 7
    }
}

// ----------------------------------------------------------------------------
// transpose / U~ waves (4, 5): chunk n+1
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void tp_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int ti = w - 4;     // value tile of U~ (0 or 1)
    const int x = tid - 256;  // 0..127
    const int l32 = lane & 31, h = lane >> 5;
    const int T = job.T;
    const size_t qk_base = (size_t)un.head * T * DK;
    const size_t v_base = (size_t)un.head * T * DV + un.r0;
    // k: keys 8jc..8jc+7 of tokens 4tg..4tg+3 and 32+4tg..32+4tg+3;
    // v: values 8vc..8vc+7 of tokens 4vt..4vt+3
    const int jc = x & 15, tg = x >> 4;
    const int vc = x & 7, vt = x >> 3;
    uint4 kr[8], vr[4], qr[8];
    auto load_q = [&](int m) {
        const Rows rq(job.q + qk_base, m, T, DK);
#pragma unroll
        for (int i = 0; i < 8; ++i) qr[i] = rq.at(32 * (i >> 2) + 4 * tg + (i & 3), 8 * jc);
    };
    auto load_raw = [&](int m) {
        const Rows rk(job.k + qk_base, m, T, DK), rv(job.v + v_base, m, T, DV);
#pragma unroll
        for (int i = 0; i < 8; ++i) kr[i] = rk.at(32 * (i >> 2) + 4 * tg + (i & 3), 8 * jc);
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = un.erows ? make_uint4(0, 0, 0, 0) : rv.at(4 * vt + i, 8 * vc);
    };
    if (un.nb < un.ne) {
        load_raw(un.nb);
        load_q(un.nb);
    }

    for (int it = un.nb - 1; it < un.ne; ++it) {
        const int m = it + 1;
        const bool act = m < un.ne;
        const int buf = m & 1;
        // ---- phase 1: k^T and v^T tiles of chunk m ----
        if (act) {
            uint16_t* KT = sm.KT[buf];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int wi = e >> 1;
                    const uint4* kk = &kr[4 * half];
                    uint2 u;
                    u.x = (e & 1) ? hi16x2(word(kk[0], wi), word(kk[1], wi)) : lo16x2(word(kk[0], wi), word(kk[1], wi));
                    u.y = (e & 1) ? hi16x2(word(kk[2], wi), word(kk[3], wi)) : lo16x2(word(kk[2], wi), word(kk[3], wi));
                    *reinterpret_cast<uint2*>(&KT[tsw(8 * jc + e, 32 * half + 4 * tg)]) = u;
                }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int wi = e >> 1;
                uint2 u;
                u.x = (e & 1) ? hi16x2(word(vr[0], wi), word(vr[1], wi)) : lo16x2(word(vr[0], wi), word(vr[1], wi));
                u.y = (e & 1) ? hi16x2(word(vr[2], wi), word(vr[3], wi)) : lo16x2(word(vr[2], wi), word(vr[3], wi));
                *reinterpret_cast<uint2*>(&sm.VT[tsw(8 * vc + e, 4 * vt)]) = u;
            }
        }
        lds_barrier();  // 1
        // ---- phase 2: next chunk's k, v in flight; diagonal 16x16 inverses 2ti, 2ti+1 ----
        if (act && m + 1 < un.ne) load_raw(m + 1);
        if (GDN && act) {
            diag_inverse(sm, 2 * ti, lane);
            diag_inverse(sm, 2 * ti + 1, lane);
        }
        lds_barrier();  // 2
        lds_barrier();  // 3
        // ---- phase 4: q tile of chunk m (the state waves read chunk n's in phases 2-3) ----
        if (act) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint4*>(&sm.Q[(32 * (i >> 2) + 4 * tg + (i & 3)) * LW + 8 * jc]) = qr[i];
            if (m + 1 < un.ne) load_q(m + 1);
        }
        lds_barrier();  // 4
        lds_barrier();  // 5
        if (GDN && act) build_tb(sm, sm.gate[buf], tid - 128);
        lds_barrier();  // 6
        // ---- phase 7: U~ = T diag(beta) V for value tile ti (gla: U~ = V) ----
        if (act) {
            if (GDN) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    f32x16 acc = {};
                    const uint16_t* tr = &sm.a.t.Tb[(32 * tt + l32) * LT + 8 * h];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        if (tt == 0 && kk >= 2) continue;
                        acc = mfma32(lds8(tr + 16 * kk), lds8(&sm.VT[tsw(32 * ti + l32, 16 * kk + 8 * h)]), acc);
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        sm.Ut[(32 * tt + 8 * (e >> 2) + 4 * h + (e & 3)) * LU + 32 * ti + l32] = acc[e];
                }
            } else {
                for (int e = x; e < C * DVS; e += 128) {
                    const int t = e >> 6, i = e & 63;
                    sm.Ut[t * LU + i] = bf16_to_f32(sm.VT[tsw(i, t)]);
                }
            }
        }
        lds_barrier();  // 7
    }
}

template <int MODE, int ROLE>
__global__ __launch_bounds__(NT, 1) void chunk_mfma_kernel(const ChunkJob job) {
    __shared__ Smem sm;
    const Unit un = unit_of<ROLE>(job);
    const int w = wave_id();
    if (w < 2)
        state_role<MODE, ROLE>(sm, job, un);
    else if (w == 4 || w == 5)
        tp_role<MODE, ROLE>(sm, job, un);
    else
        gram_role<MODE, ROLE>(sm, job, un);
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
