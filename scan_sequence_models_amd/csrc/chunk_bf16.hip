// chunk_bf16.hip -- fused bfloat16 MFMA chunk kernel (dk = dv = 128, C = 64).
//
// What it computes: the chunkwise form of the affine scan S_t = S_{t-1} E_t + f_t
// (gated delta rule: E_t = alpha_t (I - beta_t k_t k_t^T), f_t = bw_t v_t k_t^T
// with the write strength bw_t = beta_t unless erase and write are split;
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
//   W    = T diag(beta gamma) K                             WY factor   (MFMA)
//   P    = (Q K^T) * Gamma * M_incl                         scores      (MFMA)
//   U    = T diag(bw) V - W S^T                             (MFMA, needs S)
//   O    = diag(gamma) Q S^T + P U                          (MFMA, needs S)
//   S   <- gamma_C S + U^T diag(dec) K                      (MFMA, fp32 state)
//
// gated linear attention: U = V and A, T, W vanish.
//
// Mapping onto gfx950.  A workgroup of 8 waves owns one head and a 64-row slice
// of its value channels (B*H*2 workgroups on the sequential path); all slices of
// a head go to one XCD (blocks are dealt round-robin over the 8 XCDs) so their
// repeated q/k reads share that XCD's L2.  The waves specialise and work on
// three chunks at once:
//   waves 0-1      state waves: wave w keeps the 32 value columns [32w, 32w+32)
//                  of S^T (128 keys, fp32) in four 32x32 MFMA accumulator tiles
//                  for the whole sequence and runs chunk n's S-dependent
//                  products (U, O, the state update);
//   waves 2,3,6,7  chunk n+1's UT solve: the two diagonal 32x32 blocks of T
//                  are inverted inside one wave each (no barrier), the
//                  off-diagonal block by two waves, then W; one of them builds
//                  chunk n+2's off-diagonal k-Gram tile beside W;
//   waves 4-5      load chunk n+2 (coalesced 16-byte rows), stage it in LDS
//                  (q, k row-major; k^T, v^T transposed), compute its two
//                  diagonal k-Gram tiles and two of chunk n+1's score tiles.
// Everything meets through LDS and all waves pass the same three barriers per
// chunk.  Products are v_mfma_f32_32x32x16_bf16 (fp32 accumulation, bf16
// operands) except the UT solve, which stays in fp32: diagonal 16x16 blocks by
// forward substitution on the VALU, off-diagonal blocks on the fp32 MFMA
// (16x16x4).
//
// Operand trick: a 32x32 accumulator tile holds, in lane (n, h), rows
// 8b + 4h + r (b, r < 4) of column n.  Elements 8s..8s+7 of a lane are then the
// 8 rows {16s + 8b' + 4h + r}: a B operand whose contraction index is the
// tile's row.  Rows are therefore numbered with bits 2 and 3 swapped (perm5):
// accumulator row rho holds key/token perm5(rho), and elements 8s..8s+7 are the
// consecutive keys/tokens 16s + 8h .. 16s + 8h + 7.  Every LDS array whose
// rows are read as an A operand stores logical row r at physical row perm5(r),
// so that all operand reads are natural 16-byte row reads (conflict-free with
// the padded strides below).
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
constexpr int LW = DK + 8;   // row stride (elements) of [token][key] bf16 arrays
constexpr int LT = C + 8;    // row stride of [*][token] bf16 arrays
constexpr int LS = 32 + 4;   // row stride of fp32 32x32 solve tiles

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// Gates of one chunk: g = in-chunk cumulative ln alpha, gamma = e^g,
// dec = e^(g_C - g), beta (erase) and bw (write strength); gl = g log2(e) and
// gb = gl + log2(beta) feed the masks as exp2(gl_t - gl_s) = Gamma_ts and
// exp2(gb_t - gl_s) = beta_t Gamma_ts.
struct Gates {
    float g[C], gam[C], dec[C], bet[C], bw[C], gl[C], gb[C];
};

// Shared memory of one workgroup (159 KB).  Chunk c's gates live in gate[c % 3],
// its q in Q[c % 2], its k^T in KT[c % 2]; the other arrays are single.
struct Smem {
    uint16_t Q[2][C * LW];    // q [token][key]                        (rows perm5)
    uint16_t K[C * LW];       // k [token][key]                        (rows perm5)
    uint16_t W[C * LW];       // -W [token][key]                       (rows perm5)
    uint16_t KT[2][DK * LT];  // k^T [key][token]     (rows perm5, token granules swizzled)
    uint16_t VT[DVS * LT];    // v slice^T [value][token]              (token granules swizzled)
    uint16_t P[C * LT];       // scores [token][token]                 (rows perm5)
    uint16_t Tb[C * LT];      // T diag(bw) [token][token]             (rows perm5)
    uint16_t Tbg[C * LT];     // T diag(beta gamma)                    (rows perm5)
    float Tm[2][32 * LS];     // diagonal 32x32 blocks of A, then of T (fp32, natural)
    float Abl[32 * LS];       // A rows 32..63, columns 0..31 (fp32, natural)
    Gates gate[3];
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
// bf16 rounding of float vectors (packed conversions, two values per instruction)
template <int OFF>
__device__ __forceinline__ bf16x8 half8(const f32x16& x) {
    const f32x8 v = __builtin_shufflevector(x, x, OFF, OFF + 1, OFF + 2, OFF + 3, OFF + 4, OFF + 5,
                                            OFF + 6, OFF + 7);
    return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return __builtin_bit_cast(uint2, __builtin_convertvector((f32x4{a, b, c, d}), bf16x4));
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
// low (high) 16-bit halves of a and b, a's in the low half of the result
__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
__device__ __forceinline__ uint32_t word(const uint4& u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
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

// Row permutation: swap bits 2 and 3 (an involution that keeps 32-row blocks).
__device__ __forceinline__ int perm5(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// Key (state tile) or token (U / O tile) held by accumulator element e of a
// lane in half h of the wave: perm5 of the accumulator row.
__device__ __forceinline__ int elem_index(int tile, int e, int h) {
    return 32 * tile + 16 * (e >> 3) + 8 * h + 4 * ((e >> 2) & 1) + (e & 3);
}
// [row][token] arrays with 8-token granules XOR-swizzled by row, so that the
// transposed 8-byte stores spread over the LDS banks (prow: physical row).
__device__ __forceinline__ int tsw(int prow, int tok) {
    return prow * LT + ((((tok >> 3) ^ (prow >> 3)) & 7) << 3) + (tok & 7);
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
// Per-token float of chunk m (alpha or beta); tokens past T read as 0.  The
// caller substitutes any other pad value where it uses the result, so that the
// load stays in flight until then.
__device__ __forceinline__ float ldtok(const float* head, int m, int i, int T) {
    const int valid = __builtin_amdgcn_readfirstlane(min(max(T - m * C, 0), C));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(head + (size_t)m * C), (short)0, valid * 4, 0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
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

// 16x16 block products of the UT solve (fp32 MFMA 16x16x4); lane (n16, g4)
// holds rows 4 g4 .. 4 g4 + 3 of column n16 of a result.
struct Solve {
    int n16, g4;
    // acc += X Y, both 16x16 blocks of fp32 tiles with row stride LS; lane
    // (n16, g4) supplies the contraction indices 4 g4 .. 4 g4 + 3, so its X
    // operands are one 16-byte row read
    __device__ __forceinline__ f32x4 mul_lds(const float* X, const float* Y, f32x4 acc) const {
        const f32x4 xr = *reinterpret_cast<const f32x4*>(&X[n16 * LS + 4 * g4]);
        float yc[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) yc[kk] = Y[(4 * g4 + kk) * LS + n16];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma4(xr[kk], yc[kk], acc);
        return acc;
    }
    // acc += X Y, X a block in LDS, Y an accumulator block (k = 4 g4 + kk)
    __device__ __forceinline__ f32x4 mul_acc(const float* X, f32x4 Yacc, f32x4 acc) const {
        const f32x4 xr = *reinterpret_cast<const f32x4*>(&X[n16 * LS + 4 * g4]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma4(xr[kk], Yacc[kk], acc);
        return acc;
    }
    __device__ __forceinline__ void put(float* dst, f32x4 acc, float sign) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * LS + n16] = sign * acc[r];
    }
};

// In place: the two 16x16 diagonal blocks of the fp32 32x32 tile X (unit lower
// triangular I + A_bb, strictly lower part stored) are replaced by their
// inverses, by forward substitution in fp32.  Lane (b, c) (lanes 0..31; lanes
// 32..63 repeat them and store nothing) owns column c of block b's inverse:
// x_r = [r == c] - sum_{j<r} A_rj x_j (left-looking), with row r read as
// broadcast 16-byte loads issued two rows ahead.
__device__ __forceinline__ void diag_inverse2(float* X, int lane) {
    const int b = (lane >> 4) & 1, c = lane & 15;
    const float* A = X + 16 * b * LS + 16 * b;
    float x[16];
    f32x4 row[3][4];  // rows r, r+1, r+2 in flight (columns 0 .. 4*ceil(r/4)-1)
    auto load_row = [&](int r, f32x4 (&dst)[4]) {
#pragma unroll
        for (int q = 0; q < (r + 3) / 4; ++q) dst[q] = *reinterpret_cast<const f32x4*>(&A[r * LS + 4 * q]);
    };
    load_row(1, row[1]);
    load_row(2, row[2]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r + 2 < 16) load_row(r + 2, row[(r + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int q = 0; q < (r + 3) / 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * q + i;
                if (j < r) {
                    if (i & 1) s1 += row[r % 3][q][i] * x[j];
                    else s0 += row[r % 3][q][i] * x[j];
                }
            }
        x[r] = (r == c ? 1.f : 0.f) - (s0 + s1);
    }
    if (lane < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) X[(16 * b + r) * LS + 16 * b + c] = x[r];
    }
}

// acc += sum_{k < N} A(k) B(k) with the LDS operand A(k) loaded two steps
// ahead of its MFMA; the order is pinned so that each MFMA waits only for its
// own operand while the next two loads are in flight.
template <int N, typename LA, typename GB>
__device__ __forceinline__ f32x16 mfma_chain(LA load_a, GB get_b, f32x16 acc) {
    bf16x8 a0 = load_a(0), a1 = N > 1 ? load_a(1) : a0;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const bf16x8 a2 = k + 2 < N ? load_a(k + 2) : a0;
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(a0, get_b(k), acc);
        a0 = a1;
        a1 = a2;
    }
    return acc;
}

// As mfma_chain, with both operands loaded from LDS two steps ahead.
template <int N, typename LA, typename LB>
__device__ __forceinline__ f32x16 mfma_chain2(LA load_a, LB load_b, f32x16 acc) {
    bf16x8 a0 = load_a(0), b0 = load_b(0);
    bf16x8 a1 = N > 1 ? load_a(1) : a0, b1 = N > 1 ? load_b(1) : b0;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const bf16x8 a2 = k + 2 < N ? load_a(k + 2) : a0;
        const bf16x8 b2 = k + 2 < N ? load_b(k + 2) : b0;
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(a0, b0, acc);
        a0 = a1; b0 = b1;
        a1 = a2; b1 = b2;
    }
    return acc;
}

// B operand for contraction step kk (16 rows) from accumulator tiles:
// tile kk/2, elements 8(kk%2) .. 8(kk%2)+7, rounded to bf16.
template <int N>
__device__ __forceinline__ bf16x8 sop(const f32x16 (&t)[N], int kk) {
    return (kk & 1) ? half8<8>(t[kk >> 1]) : half8<0>(t[kk >> 1]);
}

// One 32x32 k-Gram or score tile of chunk-local tokens, computed transposed:
// acc[s][t] = sum_key Y[s][key] X[t][key] with s = 32J + row, t = 32I + column.
// X and Y are [token][key] LDS arrays with rows perm5, read at natural rows, so
// lane l32 holds column t = 32I + perm5(l32) and element e row
// s = 32J + elem_index(0, e, h).
__device__ __forceinline__ f32x16 gram_tile(const uint16_t* X, int I, const uint16_t* Y, int J,
                                            int l32, int h) {
    const uint16_t* xr = X + (32 * I + l32) * LW + 8 * h;
    const uint16_t* yr = Y + (32 * J + l32) * LW + 8 * h;
    return mfma_chain2<8>([&](int k) { return lds8(yr + 16 * k); },
                          [&](int k) { return lds8(xr + 16 * k); }, f32x16{});
}

// Decay mask of tile (I, J): element e of lane (l32, h) is scaled by
// e^(g_t - g_s) (times beta_t for A) where t >= s (t > s for A), else zeroed;
// tiles below the diagonal (I > J) need no comparison.  Results in the same
// layout, 4 consecutive s per element group.
template <bool IS_A>
__device__ __forceinline__ f32x16 mask_tile(const f32x16& acc, const Gates& G, int I, int J,
                                            int l32, int h) {
    const int t = 32 * I + perm5(l32);
    const float et = IS_A ? G.gb[t] : G.gl[t];
    f32x16 r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int s0 = 32 * J + elem_index(0, 4 * b, h);
        const f32x4 gs = *reinterpret_cast<const f32x4*>(&G.gl[s0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = __builtin_amdgcn_exp2f(et - gs[i]) * acc[4 * b + i];
            if (I > J) r[4 * b + i] = d;
            else r[4 * b + i] = (IS_A ? t > s0 + i : t >= s0 + i) ? d : 0.f;
        }
    }
    return r;
}

// Scores tile (I, J) of chunk m, masked, packed to bf16 (lane's row of P:
// physical row 32I + l32, columns 32J + elem_index(0, 4b, h) .. +3).
__device__ __forceinline__ void score_tile(const Smem& sm, int qbuf, const Gates& G, int I, int J,
                                           int l32, int h, uint2 (&out)[4]) {
    const f32x16 acc = gram_tile(sm.Q[qbuf], I, sm.K, J, l32, h);
    const f32x16 p = mask_tile<false>(acc, G, I, J, l32, h);
#pragma unroll
    for (int b = 0; b < 4; ++b) out[b] = pack4(p[4 * b], p[4 * b + 1], p[4 * b + 2], p[4 * b + 3]);
}
__device__ __forceinline__ void store_score_tile(Smem& sm, int I, int J, int l32, int h,
                                                 const uint2 (&p)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
        *reinterpret_cast<uint2*>(&sm.P[(32 * I + l32) * LT + 32 * J + elem_index(0, 4 * b, h)]) = p[b];
}

// k-Gram tile (I, J) of chunk m masked into A (fp32, natural indices, local to
// the 32x32 destination tile `dst`).
__device__ __forceinline__ void a_tile(const Smem& sm, const Gates& G, int I, int J, float* dst,
                                       int l32, int h) {
    const f32x16 acc = gram_tile(sm.K, I, sm.K, J, l32, h);
    const f32x16 a = mask_tile<true>(acc, G, I, J, l32, h);
    const int tl = perm5(l32);
#pragma unroll
    for (int b = 0; b < 4; ++b)
        *reinterpret_cast<f32x4*>(&dst[tl * LS + elem_index(0, 4 * b, h)]) =
            f32x4{a[4 * b], a[4 * b + 1], a[4 * b + 2], a[4 * b + 3]};
}

// Gates of chunk c from alpha, beta, bw of token `lane` (0 past T; identity
// tokens there: alpha = 1, beta = bw = 0): an inclusive wave scan of ln alpha.
__device__ __forceinline__ void stage_gates(Gates& G, int c, float pa, float pb, float pw, int T,
                                            int lane) {
    const float x = wave_inclusive_sum(c * C + lane < T ? __logf(pa) : 0.f);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    const float xl = x * 1.4426950408889634f;  // log2(e)
    G.g[lane] = x;
    G.gam[lane] = __expf(x);
    G.dec[lane] = __expf(last - x);
    G.bet[lane] = pb;
    G.bw[lane] = pw;
    G.gl[lane] = xl;
    G.gb[lane] = xl + __builtin_amdgcn_logf(pb);  // log2; -inf where beta = 0
}

struct Unit {
    int head, leaf, sl, nb, ne, r0;
    bool erows;
};

// Slices per unit: two of value rows, plus (delta rule, leaf aggregates) two of
// E's rows carried from the identity.  With gated linear attention E is
// gamma I and the tree path forms it from the gates (the E rows of a leaf
// aggregate are not written here).
template <int MODE, int ROLE>
__device__ __forceinline__ Unit unit_of(const ChunkJob& job) {
    constexpr int NS = ROLE == kLeafAggregate && MODE == 0 ? 4 : 2;
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
    constexpr bool OUT = ROLE != kLeafAggregate;  // o is read out (not for leaf aggregates)
    const int tid = threadIdx.x, lane = tid & 63, ib = wave_id();
    const int l32 = lane & 31, h = lane >> 5;
    const int T = job.T;
    const int vl = 32 * ib + l32;   // value channel of this lane within the slice
    const int vcol = un.r0 + vl;    // state row (value channel) of this lane

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

    // sbf[kk]: the state rounded to bf16 as B operands (contraction step kk);
    // qacc[tt] = Q S^T of the chunk the next iteration reads out (old state)
    bf16x8 sbf[8];
    auto round_state = [&]() {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) sbf[kk] = sop(sacc, kk);
    };
    f32x16 qacc[2];
    auto q_state = [&](int c) {
        const uint16_t* Q = sm.Q[c & 1];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const uint16_t* qr = &Q[(32 * tt + l32) * LW + 8 * h];
            qacc[tt] = mfma_chain<8>([&](int k) { return lds8(qr + 16 * k); },
                                     [&](int k) { return sbf[k]; }, f32x16{});
        }
    };
    round_state();

    lds_barrier();  // prologue: chunk nb staged
    for (int it = un.nb - 1; it < un.ne; ++it) {
        const bool act = it >= un.nb;
        const int n = it;
        const Gates& G = sm.gate[(n + 3) % 3];
        f32x16 uacc[2];
        // ---- phase A: U = T diag(beta) V - W S^T ----
        if (act) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                if (GDN) {
                    // T diag(beta) V operands read first (T is lower triangular:
                    // tile 0 contracts over tokens 0..31 only); they arrive while
                    // the W S^T chain runs
                    const uint16_t* tr = &sm.Tb[(32 * tt + l32) * LT + 8 * h];
                    bf16x8 ta[4], va[4];
                    const int nk = un.erows ? 0 : tt == 0 ? 2 : 4;  // rows of E: v = 0
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        if (kk >= nk) continue;
                        ta[kk] = lds8(tr + 16 * kk);
                        va[kk] = lds8(&sm.VT[tsw(vl, 16 * kk + 8 * h)]);
                    }
                    const uint16_t* wr = &sm.W[(32 * tt + l32) * LW + 8 * h];
                    f32x16 acc = mfma_chain<8>([&](int k) { return lds8(wr + 16 * k); },
                                               [&](int k) { return sbf[k]; }, f32x16{});
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        if (kk >= nk) continue;
                        acc = mfma32(ta[kk], va[kk], acc);
                    }
                    uacc[tt] = acc;
                } else {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const bf16x8 v8 = lds8(&sm.VT[tsw(vl, 32 * tt + 16 * s + 8 * h)]);
#pragma unroll
                        for (int i = 0; i < 8; ++i) uacc[tt][8 * s + i] = static_cast<float>(v8[i]);
                    }
                }
            }
        }
        lds_barrier();  // A
        // ---- phase B: O = diag(gamma) Q S^T + P U, written out; S^T <- gamma_C S^T + K^T diag(dec) U ----
        if (OUT && act) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x16 acc = qacc[tt];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const f32x4 g0 = *reinterpret_cast<const f32x4*>(&G.gam[32 * tt + 16 * b + 8 * h]);
                    const f32x4 g1 = *reinterpret_cast<const f32x4*>(&G.gam[32 * tt + 16 * b + 8 * h + 4]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[8 * b + i] *= g0[i];
                        acc[8 * b + 4 + i] *= g1[i];
                    }
                }
                const uint16_t* pr = &sm.P[(32 * tt + l32) * LT + 8 * h];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if (tt == 0 && ks >= 2) continue;  // P is lower triangular
                    acc = mfma32(lds8(pr + 16 * ks), sop(uacc, ks), acc);
                }
                if (job.o) {
                    // rows past T fall outside the resource and are dropped
                    const int valid = __builtin_amdgcn_readfirstlane(min(T - n * C, C));
                    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                        job.o + ((size_t)un.head * T + (size_t)n * C) * DV + un.r0, (short)0,
                        valid * DV * 2 - un.r0 * 2, 0x00020000);
                    const int voff = (8 * h * DV + vl) * 2;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[e]), orsrc, voff,
                                                              (elem_index(tt, e, 0)) * DV * 2, 0);
                }
            }
        }
        if (act) {
            bf16x8 db[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(&G.dec[16 * ks + 8 * h]);
                const f32x4 d1 = *reinterpret_cast<const f32x4*>(&G.dec[16 * ks + 8 * h + 4]);
                const f32x16& u = uacc[ks >> 1];
                const int off = 8 * (ks & 1);
                f32x8 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = u[off + i] * d0[i];
                    x[4 + i] = u[off + 4 + i] * d1[i];
                }
                db[ks] = __builtin_convertvector(x, bf16x8);
            }
            const float gC = G.gam[C - 1];
            const uint16_t* KT = sm.KT[n & 1];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int prow = 32 * jt + l32;
                sacc[jt] = mfma_chain<4>([&](int k) { return lds8(&KT[tsw(prow, 16 * k + 8 * h)]); },
                                         [&](int k) { return db[k]; }, sacc[jt] * gC);
            }
            round_state();
        }
        lds_barrier();  // B
        // ---- phase C: Q S^T of chunk n+1 with the state entering it ----
        if (OUT && n + 1 < un.ne) q_state(n + 1);
        lds_barrier();  // C
    }

    float* dst = nullptr;
    if (ROLE == kSequential && job.S_out) dst = job.S_out + ((size_t)un.head * DV + vcol) * DK;
    if (ROLE == kLeafAggregate)
        dst = job.S_out + ((size_t)(un.head * job.leaves + un.leaf) * (DV + DK) + un.sl * DVS + vl) * DK;
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

// ----------------------------------------------------------------------------
// k-Gram / UT solve / W waves (2, 3, 6, 7 -> gi 0..3): chunk n+1
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void gram_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    constexpr bool OUT = ROLE != kLeafAggregate;  // scores needed only where o is read out
    const int lane = threadIdx.x & 63, w = wave_id();
    const int gi = w == 2 ? 0 : w == 3 ? 1 : w == 6 ? 2 : 3;
    const int l32 = lane & 31, h = lane >> 5;
    const Solve sv{lane & 15, lane >> 4};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    uint2 preg[4];  // gi 3: chunk m's score tile (1, 0), stored in phase C
    // gi 0: alpha, beta of chunk m+1's token `lane` (0 past T); its gates
    const int T = job.T;
    const size_t a_base = (size_t)un.head * T;
    float pa = 1.f, pb = 0.f, pw = 0.f;
    const bool split = job.beta_w != job.beta;  // separate write strengths
    auto load_ab = [&](int c) {
        pa = ldtok(job.alpha + a_base, c, lane, T);
        if (GDN) {
            pb = ldtok(job.beta + a_base, c, lane, T);
            if (split) pw = ldtok(job.beta_w + a_base, c, lane, T);
        }
    };
    if (gi == 0 && un.nb < un.ne) {
        load_ab(un.nb);
        stage_gates(sm.gate[un.nb % 3], un.nb, pa, pb, split ? pw : pb, T, lane);
    }

    lds_barrier();  // prologue
    for (int it = un.nb - 1; it < un.ne; ++it) {
        const int m = it + 1;
        const bool act = m < un.ne;
        const Gates& G = sm.gate[m % 3];
        // ---- phase A: diagonal 32x32 blocks of T in-wave (the first chunk also builds its k-Gram tiles) ----
        if (gi == 0 && m + 1 < un.ne) load_ab(m + 1);
        if (act) {
            if (GDN && gi <= 1) {
                float* X = sm.Tm[gi];
                // later chunks' diagonal tiles come from the load waves (phase C)
                if (m == un.nb) a_tile(sm, G, gi, gi, X, l32, h);
                diag_inverse2(X, lane);
                // T_10 = -D_1 A_10 D_0 within the 32x32 block
                const f32x4 mm = sv.mul_lds(X + 16 * LS, X, z);
                sv.put(X + 16 * LS, sv.mul_acc(X + 16 * LS + 16, mm, z), -1.f);
            } else if (GDN && gi == 2) {
                // later chunks' tile is built in the previous phase C
                if (m == un.nb) a_tile(sm, G, 1, 0, sm.Abl, l32, h);
            } else if (OUT && gi == 3) {
                score_tile(sm, m & 1, G, 1, 0, l32, h, preg);
            }
        }
        lds_barrier();  // A
        // ---- phase B: off-diagonal 32x32 block of T; bf16 Tb = T diag(bw), Tbg = T diag(beta gamma) ----
        if (GDN && act) {
            if (gi <= 1) {
                // rows 32gi + tl of the diagonal block, 16 columns from c0
                const float* X = sm.Tm[gi];
                const int tl = lane >> 1, c0 = 16 * (lane & 1);
                const int prow = 32 * gi + perm5(tl);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    uint32_t b[4], bg[4];
                    const int s0 = 32 * gi + c0 + 8 * hh;
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(&X[tl * LS + c0 + 8 * hh]);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(&X[tl * LS + c0 + 8 * hh + 4]);
                    const f32x4 be0 = *reinterpret_cast<const f32x4*>(&G.bet[s0]);
                    const f32x4 be1 = *reinterpret_cast<const f32x4*>(&G.bet[s0 + 4]);
                    const f32x4 bw0 = *reinterpret_cast<const f32x4*>(&G.bw[s0]);
                    const f32x4 bw1 = *reinterpret_cast<const f32x4*>(&G.bw[s0 + 4]);
                    const f32x4 ga0 = *reinterpret_cast<const f32x4*>(&G.gam[s0]);
                    const f32x4 ga1 = *reinterpret_cast<const f32x4*>(&G.gam[s0 + 4]);
                    float tv[8], bv[8], wv[8], gv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tv[i] = x0[i]; tv[4 + i] = x1[i];
                        bv[i] = be0[i]; bv[4 + i] = be1[i];
                        wv[i] = bw0[i]; wv[4 + i] = bw1[i];
                        gv[i] = ga0[i]; gv[4 + i] = ga1[i];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int sa = c0 + 8 * hh + 2 * i;  // local column of element 2i
                        const float t0 = sa <= tl ? tv[2 * i] : 0.f;
                        const float t1 = sa + 1 <= tl ? tv[2 * i + 1] : 0.f;
                        b[i] = pack2(t0 * wv[2 * i], t1 * wv[2 * i + 1]);
                        bg[i] = pack2(t0 * bv[2 * i] * gv[2 * i], t1 * bv[2 * i + 1] * gv[2 * i + 1]);
                    }
                    *reinterpret_cast<uint4*>(&sm.Tb[prow * LT + s0]) = make_uint4(b[0], b[1], b[2], b[3]);
                    *reinterpret_cast<uint4*>(&sm.Tbg[prow * LT + s0]) = make_uint4(bg[0], bg[1], bg[2], bg[3]);
                }
            } else {
                // columns 16J .. 16J+15 of T rows 32..63:
                //   Y_iJ = sum_K A_bl(i, K) T_0(K, J),  T_bl(i, J) = -sum_K T_1(i, K) Y_KJ
                const int J = gi - 2;
                const float* T0 = sm.Tm[0];
                const float* T1 = sm.Tm[1];
                f32x4 y0, y1;
                if (J == 0) {
                    y0 = sv.mul_lds(sm.Abl + 16, T0 + 16 * LS, sv.mul_lds(sm.Abl, T0, z));
                    y1 = sv.mul_lds(sm.Abl + 16 * LS + 16, T0 + 16 * LS, sv.mul_lds(sm.Abl + 16 * LS, T0, z));
                } else {
                    y0 = sv.mul_lds(sm.Abl + 16, T0 + 16 * LS + 16, z);
                    y1 = sv.mul_lds(sm.Abl + 16 * LS + 16, T0 + 16 * LS + 16, z);
                }
                const f32x4 t0 = sv.mul_acc(T1, y0, z);
                const f32x4 t1 = sv.mul_acc(T1 + 16 * LS + 16, y1, sv.mul_acc(T1 + 16 * LS, y0, z));
                const int s = 16 * J + sv.n16;
                const float bs = G.bw[s], bgs = G.bet[s] * G.gam[s];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p0 = 32 + perm5(4 * sv.g4 + r), p1 = 32 + perm5(16 + 4 * sv.g4 + r);
                    sm.Tb[p0 * LT + s] = f32_to_bf16(-t0[r] * bs);
                    sm.Tbg[p0 * LT + s] = f32_to_bf16(-t0[r] * bgs);
                    sm.Tb[p1 * LT + s] = f32_to_bf16(-t1[r] * bs);
                    sm.Tbg[p1 * LT + s] = f32_to_bf16(-t1[r] * bgs);
                }
            }
        }
        // chunk m+1's gates: the load waves mask its k-Gram tiles in phase C
        if (gi == 0 && m + 1 < un.ne)
            stage_gates(sm.gate[(m + 1) % 3], m + 1, pa, pb, split ? pw : pb, T, lane);
        lds_barrier();  // B
        // ---- phase C: W = T diag(beta gamma) K (stored -W): key tile gi, and tile 2 on
        // gi 1; gi 2 builds chunk m+1's off-diagonal k-Gram tile; scores ----
        auto w_tile = [&](int jt) {
            const uint16_t* KT = sm.KT[m & 1];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint16_t* tr = &sm.Tbg[(32 * tt + l32) * LT + 8 * h];
                auto lk = [&](int k) { return lds8(&KT[tsw(32 * jt + l32, 16 * k + 8 * h)]); };
                auto lt = [&](int k) { return lds8(tr + 16 * k); };
                // T is lower triangular: token tile 0 needs columns 0..31 only
                const f32x16 acc = tt == 0 ? mfma_chain2<2>(lk, lt, f32x16{}) : mfma_chain2<4>(lk, lt, f32x16{});
                uint16_t* wrow = &sm.W[(32 * tt + l32) * LW + 32 * jt];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    *reinterpret_cast<uint2*>(wrow + elem_index(0, 4 * b, h)) =
                        pack4(-acc[4 * b], -acc[4 * b + 1], -acc[4 * b + 2], -acc[4 * b + 3]);
            }
        };
        if (act) {
            if (GDN) {
                if (gi != 2) w_tile(gi);
                if (gi == 1) w_tile(2);
                if (gi == 2 && m + 1 < un.ne) a_tile(sm, sm.gate[(m + 1) % 3], 1, 0, sm.Abl, l32, h);
            }
            if (OUT && gi == 3) store_score_tile(sm, 1, 0, l32, h, preg);
        }
        lds_barrier();  // C
    }
}

// ----------------------------------------------------------------------------
// load / transpose waves (4, 5): stage chunk n+2 and its diagonal k-Gram
// tiles; score tiles (0,0), (1,1) of n+1
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void tp_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    constexpr bool OUT = ROLE != kLeafAggregate;  // q and scores needed only where o is read out
    // The roles share one control-flow graph, so the compiler's wait-count
    // analysis can take another role's loads as still in flight here and wait
    // for every load at each reuse of their registers inside the loop below.
    // An explicit vmcnt(0) (free: this wave has issued no load yet) clears that.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int ti = w - 4;     // score tile (ti, ti)
    const int x = tid - 256;  // 0..127
    const int l32 = lane & 31, h = lane >> 5;
    const int T = job.T;
    const size_t qk_base = (size_t)un.head * T * DK;
    const size_t v_base = (size_t)un.head * T * DV + un.r0;
    // q, k: keys 8jc..8jc+7 of tokens 32(i>>2) + 4tg + (i&3), i < 8;
    // v: values 8vc..8vc+7 of tokens 4vt + i, i < 4
    const int jc = x & 15, tg = x >> 4;
    const int vc = x & 7, vt = x >> 3;
    uint4 qr[8], kc[8], kn[8], vcur[4], vnx[4];
    auto load = [&](int c, uint4 (&kk)[8], uint4 (&vv)[4]) {
        const Rows rq(job.q + qk_base, c, T, DK), rk(job.k + qk_base, c, T, DK), rv(job.v + v_base, c, T, DV);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 32 * (i >> 2) + 4 * tg + (i & 3);
            kk[i] = rk.at(row, 8 * jc);
            if (OUT) qr[i] = rq.at(row, 8 * jc);
        }
        if (un.erows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = make_uint4(0, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = rv.at(4 * vt + i, 8 * vc);
        }
    };
    // k, q rows of chunk c (from kk, qr) and its gates into LDS
    auto stage = [&](int c, const uint4 (&kk)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int prow = perm5(32 * (i >> 2) + 4 * tg + (i & 3));
            *reinterpret_cast<uint4*>(&sm.K[prow * LW + 8 * jc]) = kk[i];
            if (OUT) *reinterpret_cast<uint4*>(&sm.Q[c & 1][prow * LW + 8 * jc]) = qr[i];
        }
    };
    // k^T of chunk c (from kk) into KT[c % 2]: keys 8jc + e, tokens 32half + 4tg .. +3
    auto stage_kt = [&](int c, const uint4 (&kk)[8]) {
        uint16_t* KT = sm.KT[c & 1];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int wi = e >> 1;
                const uint4* k4 = &kk[4 * half];
                uint2 u;
                u.x = (e & 1) ? hi16x2(word(k4[0], wi), word(k4[1], wi)) : lo16x2(word(k4[0], wi), word(k4[1], wi));
                u.y = (e & 1) ? hi16x2(word(k4[2], wi), word(k4[3], wi)) : lo16x2(word(k4[2], wi), word(k4[3], wi));
                *reinterpret_cast<uint2*>(&KT[tsw(perm5(8 * jc + e), 32 * half + 4 * tg)]) = u;
            }
    };
    // v^T of the chunk (from vv) into VT: values 8vc + e, tokens 4vt .. 4vt+3
    auto stage_vt = [&](const uint4 (&vv)[4]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int wi = e >> 1;
            uint2 u;
            u.x = (e & 1) ? hi16x2(word(vv[0], wi), word(vv[1], wi)) : lo16x2(word(vv[0], wi), word(vv[1], wi));
            u.y = (e & 1) ? hi16x2(word(vv[2], wi), word(vv[3], wi)) : lo16x2(word(vv[2], wi), word(vv[3], wi));
            *reinterpret_cast<uint2*>(&sm.VT[tsw(8 * vc + e, 4 * vt)]) = u;
        }
    };

    // prologue: chunk nb's k, q, gates in LDS; its k, v kept for k^T / v^T
    if (un.nb < un.ne) {
        load(un.nb, kc, vcur);
        stage(un.nb, kc);
    }
    lds_barrier();  // prologue
    uint2 preg[4];
    // one chunk step; kc/vcur hold chunk m's k and v, kn/vnx receive chunk m+1's
    auto step = [&](int it, uint4 (&kcur)[8], uint4 (&knext)[8], uint4 (&vcu)[4], uint4 (&vne)[4]) {
        const int m = it + 1;
        const bool act = m < un.ne;
        const bool nxt = m + 1 < un.ne;
        const Gates& G = sm.gate[m % 3];
        // Every load of this wave is a chunk old here; stating so keeps the
        // compiler from waiting on the loads issued just below (its analysis
        // loses track of the older ones across the conditional steps).
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // ---- phase A: chunk m+1 in flight; k^T of chunk m; score tile (ti, ti) of m ----
        if (act) {
            if (nxt) load(m + 1, knext, vne);
            stage_kt(m, kcur);
            if (OUT) score_tile(sm, m & 1, G, ti, ti, l32, h, preg);
        }
        lds_barrier();  // A
        // ---- phase B: v^T of chunk m; k, q of chunk m+1 ----
        if (act) stage_vt(vcu);
        if (nxt) stage(m + 1, knext);
        lds_barrier();  // B
        // ---- phase C: scores of m; diagonal k-Gram tile (ti, ti) of chunk m+1 ----
        if (act && OUT) store_score_tile(sm, ti, ti, l32, h, preg);
        if (GDN && nxt) a_tile(sm, sm.gate[(m + 1) % 3], ti, ti, sm.Tm[ti], l32, h);
        lds_barrier();  // C
    };
    // two steps per trip so that the current / next register sets alternate
    // without copies
    for (int it = un.nb - 1; it < un.ne; it += 2) {
        step(it, kc, kn, vcur, vnx);
        if (it + 1 < un.ne) step(it + 1, kn, kc, vnx, vcur);
    }
}

template <int MODE, int ROLE>
__global__ __launch_bounds__(NT, 1) void chunk_mfma_kernel(const ChunkJob job) {
    __shared__ Smem sm;
    const Unit un = unit_of<MODE, ROLE>(job);
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
    else if (role == kLeafAggregate) {
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kLeafAggregate>), dim3((MODE == 0 ? 4 : 2) * units), block, 0,
                           stream, job);
    }
    else
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kLeafOutput>), dim3(2 * units), block, 0, stream, job);
    return hipGetLastError();
}

hipError_t launch_chunk_job(int mode, int role, const ChunkJob& job, hipStream_t stream) {
    return mode == 0 ? launch_role<0>(role, job, stream) : launch_role<1>(role, job, stream);
}

hipError_t launch_chunk_mfma(int mode, int BH, int T, int dk, int dv, int chunk, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta,
                             const float* beta_w, const float* S0, void* o, float* ST,
                             hipStream_t stream) {
    (void)dk; (void)dv; (void)chunk;
    ChunkJob job{};
    job.q = static_cast<const uint16_t*>(q);
    job.k = static_cast<const uint16_t*>(k);
    job.v = static_cast<const uint16_t*>(v);
    job.alpha = alpha;
    job.beta = beta;
    job.beta_w = beta_w;
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
