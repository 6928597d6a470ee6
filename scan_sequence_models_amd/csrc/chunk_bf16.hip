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
//   T    = (I + A)^-1                                       UT solve
//   X    = K S^T                                            (MFMA, needs S)
//   U    = T diag(bw) V - T diag(beta gamma) X              (MFMA)
//   P    = (Q K^T) * Gamma * M_incl                         scores      (MFMA)
//   O    = diag(gamma) Q S^T + P U                          (MFMA, needs S)
//   S   <- gamma_C S + U^T diag(dec) K                      (MFMA, fp32 state)
//
// U = T (diag(bw) V - diag(beta gamma) K S^T) is the WY form's U with the
// factor W = T diag(beta gamma) K never formed; gated linear attention has
// U = V and no A, T, X.  T is applied by block forward substitution over the
// chunk's two 32-token halves: with D_0, D_1 the inverses of the diagonal blocks
// of I + A, A_bl its lower-left block and Y = diag(bw) V - diag(beta gamma) X,
// U_top = D_0 Y_top and U_bot = D_1 Y_bot + G U_top, G = -D_1 A_bl.
//
// Mapping onto gfx950.  A workgroup of 8 waves owns one head and a 64-row slice
// of its value channels (B*H*2 workgroups on the sequential path); all slices of
// a head go to one XCD (blocks are dealt round-robin over the 8 XCDs) so their
// repeated q/k reads share that XCD's L2.  The waves specialise; wave w runs on
// SIMD w % 4, and each chunk step has two halves separated by LDS barriers.  In
// step j, chunk j is read out:
//
//   waves 0, 1  state: wave w keeps the 32 value columns [32w, 32w+32) of S^T
//               (128 keys, fp32) in four 32x32 MFMA accumulator tiles for the
//               whole sequence.  First half: X = K S^T and Q S^T of chunk j;
//               second half: U, O (staged in LDS) and the state update.
//   waves 4, 5  first half: o of chunk j-1 stored from LDS (16-byte stores),
//               and the two diagonal blocks D_0, D_1 of chunk j scaled into the
//               bf16 factors Tb = D diag(bw), Tbn = -D diag(beta gamma);
//               second half: chunk j+1's q and v (and, with gated linear
//               attention, k) staged in LDS, then chunk j+2's rows loaded into
//               registers (coalesced 16-byte loads).
//   wave 2      first half: chunk j+1's two diagonal k-Gram tiles; second
//               half: the gates of chunk j+2 (a wave scan of ln alpha).
//   wave 3      first half: chunk j's score tile (0,0); second half: chunk
//               j+1's off-diagonal k-Gram tile, then (delta rule) chunk j+1's k
//               rows staged in LDS from the registers that tile read.
//   wave 6      first half: G = -D_1 A_bl of chunk j by a split-bf16 product
//               (hi/lo parts, three MFMAs per product), stored as bf16 in
//               Tb's lower-left block; second half: D_0 of chunk j+1 (16x16
//               blocks by forward substitution, the block below their
//               diagonal on the fp32 MFMA).
//   wave 7      first half: chunk j's score tiles (1,0) and (1,1); second half:
//               D_1 of chunk j+1.
//
// The k-Gram waves read k straight from global memory into MFMA operand
// registers (a chunk ahead); the other products read LDS.  Operands contracted
// over tokens (k for the state update, v for T V) come from row-major tiles
// through ds_read_b64_tr_b16 transposed reads.  LDS strides: q rows 136
// elements (16-row 16-byte reads conflict-free), k rows 160 with 16-byte
// granules XOR-swizzled by (row / 4) mod 4 (conflict-free for both 16-row
// reads and 4-row transposed reads), v rows 96 (transposed reads only), the
// [token][token] bf16 tiles 72.
//
// Operand trick: a 32x32 accumulator tile holds, in lane (n, h), rows
// 8b + 4h + r (b, r < 4) of column n.  Elements 8s..8s+7 of a lane are then the
// 8 rows {16s + 8b' + 4h + r}: a B operand whose contraction index is the
// tile's row.  Rows are therefore numbered with bits 2 and 3 swapped (perm5):
// accumulator row rho holds key/token perm5(rho), and elements 8s..8s+7 are the
// consecutive keys/tokens 16s + 8h .. 16s + 8h + 7.  Every LDS array whose
// rows are read as an A operand stores logical row r at physical row perm5(r).
//
// Tokens past T in the last chunk are identity tokens (alpha = 1, beta = 0,
// q = k = v = 0), which leave S unchanged; their outputs are not written.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int C = 64;        // tokens per chunk
constexpr int DK = 128;      // key channels
constexpr int DV = 128;      // value channels
constexpr int DVS = 64;      // value channels per workgroup
constexpr int NT = 512;      // 8 waves
constexpr int LK = 160;      // row stride (elements) of k [token][key], granules swizzled
constexpr int LQ = DK + 8;   // row stride of q [token][key]
constexpr int LV = 96;       // row stride of the v slice [token][value]
constexpr int LT = C + 8;    // row stride of [token][token] bf16 tiles
constexpr int LS = 32 + 4;   // row stride of fp32 32x32 tiles
constexpr int LO = DVS + 8;  // row stride of the staged o tile [token][value]

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Gates of one chunk: gamma = e^g, dec = e^(g_C - g), bw (write strength),
// bg = beta gamma; gl = g log2(e) and gb = gl + log2(beta) feed the masks as
// exp2(gl_t - gl_s) = Gamma_ts and exp2(gb_t - gl_s) = beta_t Gamma_ts.  When
// the chunk's log2 decay spans at most kSpan (`fast`, every factor below stays
// within 2^+-kSpan):
//  - the k-Gram mask uses the factored form beta_t Gamma_ts = ebt_t fl_s with
//    el = exp2(gl - gl_32), fl = exp2(gl_32 - gl), ebt = beta el (two
//    multiplies per element instead of an exponential);
//  - dec is folded into the rows of T's factors (and G becomes
//    diag(dec_bot) G diag(ec_top), which keeps its magnitude: the decays cancel),
//    so that U' = diag(dec) U comes out of the products and feeds the state
//    update directly, and the scores
//    become P'_ts = ec_t (q_t . k_s) with ec = exp2(gl - gl_C): P' U' = P U
//    because Gamma_ts = ec_t dec_s.
// Otherwise the exponentials of differences are taken per element and U is
// scaled by dec on the vector units.
constexpr float kSpan = 100.f;
struct alignas(16) Gates {
    float gam[C], dec[C], bw[C], bg[C], gl[C], gb[C], fl[C], ebt[C], ec[C];
    int fast, pad[3];  // (16-byte size: every slot's arrays take 16-byte reads)
};
static_assert(sizeof(Gates) % 16 == 0, "gate slots must stay 16-byte aligned");

// Shared memory of one workgroup (152 KB).  Chunk c's k and v live in slot
// c % 2 (so do the off-diagonal k-Gram tiles), its gates in slot c % 3; the
// other arrays are single.
struct Smem {
    uint16_t K[2][C * LK];    // k [token][key]                 (rows perm5, granules swizzled)
    uint16_t Q[C * LQ];       // q [token][key]                 (rows perm5)
    uint16_t V[2][C * LV];    // v slice [token][value]         (natural rows)
    uint16_t Tb[C * LT];      // T diag(bw) [token][token]      (rows perm5)
    uint16_t Tbn[C * LT];     // -T diag(beta gamma)            (rows perm5)
    uint16_t P[C * LT];       // scores [token][token]          (rows perm5)
    float At[2][32 * LS];     // diagonal k-Gram tiles of A, transposed: At[b][s][t] = A[32b+t][32b+s]
    float Ablt[2][32 * LS];   // A rows 32..63, columns 0..31, transposed
    float D[2][32 * LS];      // diagonal 32x32 blocks of T (natural)
    uint16_t Ost[C * LO];     // o of the chunk just read out [token][value] (natural rows)
    Gates gate[3];
    int ezero[2];             // leaf aggregates, rows of E: state wave w's state is exactly zero
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
__device__ __forceinline__ uint4 pack8(const f32x8& x) {
    return __builtin_bit_cast(uint4, __builtin_convertvector(x, bf16x8));
}
// Workgroup barrier that orders LDS traffic only.  __syncthreads() also waits
// for every outstanding global load and store of the wave (vmcnt), which would
// stall on prefetches and output stores at every barrier.  The memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Completes this wave's own LDS accesses before the ones that follow (a wave
// reading back what its other lanes wrote).
__device__ __forceinline__ void lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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
// Element offset of column `col` of physical row `prow` in the k tile: 16-byte
// granules XOR-swizzled by (prow / 4) mod 4.
__device__ __forceinline__ int kidx(int prow, int col) {
    return prow * LK + ((((col >> 3) ^ (prow >> 2)) & 3) | ((col >> 3) & ~3)) * 8 + (col & 7);
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
// PRISM's element stream read in place (role kPrism).  Element e = t G + l
// (G = L + 1) is token t's gated-delta element (l = 0: k_t, v_t, alpha_t,
// erase and write beta_t) or its l-th correction (k and v from the factor rows,
// alpha 1, erase 0, write beta_l[t][l-1]); q_t sits on element t G + L, whose
// output is o_t.  Elements past the stream read as identity elements.
// Every field is read with buffer loads from each of its possible sources: the
// unused source gets an offset past its resource, which the hardware returns as
// zero without a memory access.  (One load from a per-lane pointer would need
// 64-bit address arithmetic per row, which costs more than the second load.)
// The parts are merged (OR, sum) only where the value is used, half a step or
// more after the loads, so that no wait lands on the loads themselves.
struct PrismSrc {
    static constexpr unsigned kOut = 0x80000000u;  // an offset past every resource
    __amdgpu_buffer_rsrc_t q, k, v, kf, vf, alpha, beta, beta_l, o;
    int L, G, E;
    unsigned magic;
    __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    }
    __device__ __forceinline__ PrismSrc(const ChunkJob& job, int head, int r0) {
        L = job.prism_L;
        G = L + 1;
        E = job.T;
        magic = job.prism_magic;
        const size_t T = job.prism_T, tk = (size_t)head * T;
        q = rsrc(job.q + tk * DK, T * DK * 2);
        k = rsrc(job.k + tk * DK, T * DK * 2);
        v = rsrc(job.v + tk * DV + r0, T * DV * 2 - r0 * 2);
        kf = rsrc(job.kf + tk * L * DK, T * L * DK * 2);
        vf = rsrc(job.vf + tk * L * DV + r0, T * L * DV * 2 - r0 * 2);
        alpha = rsrc(job.alpha + tk, T * 4);
        beta = rsrc(job.beta + tk, T * 4);
        beta_l = rsrc(job.beta_l + tk * L, T * L * 4);
        o = rsrc(job.o ? job.o + tk * DV + r0 : job.q, job.o ? T * DV * 2 - r0 * 2 : 0);
    }
    // token t and step l of element e
    __device__ __forceinline__ void at(int e, int& t, int& l) const {
        t = (int)__umulhi((unsigned)e, magic);
        l = e - t * G;
    }
    // Byte offsets of the rows (ld elements) of element e in its token source
    // (a) and in its factor-row source (b), kOut where unused; a column's bytes
    // are added to them (offsets past the resource stay past it).
    __device__ __forceinline__ void rows(int e, int ld, unsigned& a, unsigned& b) const {
        int t, l;
        at(e, t, l);
        const bool in = e < E;
        a = in && l == 0 ? (unsigned)(t * ld) * 2 : kOut;
        b = in && l != 0 ? (unsigned)((t * L + l - 1) * ld) * 2 : kOut;
    }
    __device__ __forceinline__ unsigned q_rows(int e) const {
        int t, l;
        at(e, t, l);
        return e < E && l == L ? (unsigned)(t * DK) * 2 : kOut;
    }
    __device__ __forceinline__ static uint4 ld(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    __device__ __forceinline__ static float ldf(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    // the raw gate loads of element e: alpha (token elements), beta (token
    // elements) and beta_l (corrections), zero where unused; gates_of merges them
    __device__ __forceinline__ void gate_loads(int e, float& a, float& b, float& bl) const {
        int t, l;
        at(e, t, l);
        const bool in = e < E;
        const unsigned o0 = in && l == 0 ? (unsigned)t * 4 : kOut;
        a = ldf(alpha, o0);
        b = ldf(beta, o0);
        bl = ldf(beta_l, in && l != 0 ? (unsigned)(t * L + l - 1) * 4 : kOut);
    }
    // alpha, erase and write strength from the raw loads
    __device__ __forceinline__ void gates_of(int e, float a, float b, float bl, float& pa, float& pb,
                                             float& pw) const {
        int t, l;
        at(e, t, l);
        pa = e < E && l == 0 ? a : 1.f;
        pb = b;
        pw = b + bl;  // one of the two is zero
    }
    // o_t from element e's output row (dropped unless e is a token's last element)
    __device__ __forceinline__ void store_o(int e, int col, uint4 val) const {
        int t, l;
        at(e, t, l);
        const unsigned off = e < E && l == L ? (unsigned)(t * DV) * 2 : kOut;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, val), o, (int)(off + col * 2), 0, 0);
    }
};
__device__ __forceinline__ uint4 orv(uint4 a, uint4 b) {
    return make_uint4(a.x | b.x, a.y | b.y, a.z | b.z, a.w | b.w);
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

// MFMA operand contracted over the tokens of the v slice (natural rows): lane
// (m = lane % 32, g = lane / 32) gets tokens 16 kk + 8 g .. +7 of value
// column col0 + perm5(m), by two ds_read_b64_tr_b16 (in each 16-lane group,
// lane l receives element l % 4 of the 8-byte pieces that lanes 4 i + l / 4
// address, i = 0..3: four consecutive rows of one column; the supplied column
// swaps the two bits of the 4-value piece index, which perm5's the columns).
__device__ __forceinline__ bf16x8 v_operand(const uint16_t* V, int kk, int col0, int lane) {
    const int l = lane & 15, grp = lane >> 4;
    const int r = 16 * kk + 8 * (grp >> 1) + (l >> 2);
    const int piece = ((l & 1) << 1) | ((l >> 1) & 1);
    const int c = col0 + 16 * (grp & 1) + 4 * piece;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(V + r * LV + c));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(V + (r + 4) * LV + c));
    const s16x4 ab[2] = {a, b};
    return __builtin_bit_cast(bf16x8, ab);
}
// A operand of the state update, (K^T)[key][token], from the k tile (rows
// perm5): lane (m = lane % 32, g = lane / 32) gets key 32 jt + perm5(m) of
// tokens 16 kk + 8 g .. +7.  Token 16kk + 8g + i sits in physical row
// 16kk + 4g + i (i < 4) or 16kk + 8 + 4g + (i - 4); the supplied column swaps
// the two bits of the 4-key piece index so that the keys come out perm5'd.
__device__ __forceinline__ bf16x8 kt_operand(const uint16_t* K, int kk, int jt, int lane) {
    const int l = lane & 15, grp = lane >> 4, g = grp >> 1;
    const int r = 16 * kk + 4 * g + (l >> 2);
    const int piece = ((l & 1) << 1) | ((l >> 1) & 1);
    const int c = 32 * jt + 16 * (grp & 1) + 4 * piece;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(K + kidx(r, c)));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(K + kidx(r + 8, c)));
    const s16x4 ab[2] = {a, b};
    return __builtin_bit_cast(bf16x8, ab);
}

// hi + lo split of 8 floats into two bf16 vectors (hi = RNE(x), lo = RNE(x - hi)).
__device__ __forceinline__ void split8(const f32x8& x, bf16x8& hi, bf16x8& lo) {
    hi = __builtin_convertvector(x, bf16x8);
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8), bf16x8);
}
__device__ __forceinline__ f32x8 ld8f(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// acc += X Y in split bf16 (X_hi Y_hi + X_hi Y_lo + X_lo Y_hi)
__device__ __forceinline__ f32x16 mfma_split(const f32x8& x, const f32x8& y, f32x16 acc) {
    bf16x8 xh, xl, yh, yl;
    split8(x, xh, xl);
    split8(y, yh, yl);
    acc = mfma32(xh, yh, acc);
    acc = mfma32(xh, yl, acc);
    return mfma32(xl, yh, acc);
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
    constexpr bool EROWS = ROLE == kLeafAggregate && MODE == 0;
    const int units = job.heads * job.leaves;
    int u, sl;
    int x = blockIdx.x;
    // With rows of E (slices 2, 3), the grid holds all of them first and the
    // value rows (slices 0, 1) after: rows of E can stop early (erows_done),
    // and the value rows then start on the CUs they free instead of waiting
    // for a whole round of value rows.
    int base = 0;
    if (EROWS) {
        if (x < 2 * units) {
            base = 2;
        } else {
            x -= 2 * units;
        }
    }
    if ((units & 7) == 0) {
        const int xcd = x & 7, j = x >> 3;
        u = (j / 2) * 8 + xcd;
        sl = base + j % 2;
    } else {
        u = x / 2;
        sl = base + x % 2;
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

// Rows of E in a leaf aggregate carry S_t = S_{t-1} E_t from the identity with
// v = 0.  Once that state is exactly zero it stays zero: X = K S^T = 0, so
// U = 0 and the update only scales it (exact for finite inputs; a NaN state
// never reads as zero).  A long leaf with decaying gates gets there well before
// its end: the state waves then report it (ezero), and every wave leaves the
// chunk loop at the top of the next step, all at the same barrier count.  The
// zeros already in the state are the aggregate's rows.
template <int ROLE>
__device__ __forceinline__ bool erows_done(const Smem& sm, const Unit& un, int j) {
    if constexpr (ROLE != kLeafAggregate) {
        return false;
    } else {
        return un.erows && j > un.nb && (sm.ezero[0] & sm.ezero[1]) != 0;
    }
}

// Gates of chunk c from alpha, beta, bw of token `lane` (0 past T; identity
// tokens there: alpha = 1, beta = bw = 0): an inclusive wave scan of ln alpha.
struct LaneGates {
    float gam, dec, bw, bg, gl, gb, el, fl, ebt, ec;
    bool fast;
};
__device__ __forceinline__ LaneGates lane_gates(int c, float pa, float pb, float pw, int T, int lane) {
    const float x = wave_inclusive_sum(c * C + lane < T ? __logf(pa) : 0.f);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    LaneGates g;
    g.gl = x * 1.4426950408889634f;  // log2(e)
    g.gam = __expf(x);
    g.dec = __expf(last - x);
    g.bw = pw;
    g.bg = pb * g.gam;
    g.gb = g.gl + __builtin_amdgcn_logf(pb);  // log2; -inf where beta = 0
    const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g.gl), 0));
    const float g63 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g.gl), 63));
    const float ref = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g.gl), 32));
    g.fast = g0 - g63 <= kSpan;  // false for NaN or infinite decays
    g.el = __builtin_amdgcn_exp2f(g.gl - ref);
    g.fl = __builtin_amdgcn_exp2f(ref - g.gl);
    g.ebt = pb * g.el;
    g.ec = __builtin_amdgcn_exp2f(g.gl - g63);
    return g;
}

// Gates of chunk c into slot G (one token per lane).
__device__ __forceinline__ void form_gates(Gates& G, int c, float pa, float pb, float pw, int T, int lane) {
    const LaneGates g = lane_gates(c, pa, pb, pw, T, lane);
    G.gam[lane] = g.gam;
    G.dec[lane] = g.dec;
    G.bw[lane] = g.bw;
    G.bg[lane] = g.bg;
    G.gl[lane] = g.gl;
    G.gb[lane] = g.gb;
    G.fl[lane] = g.fl;
    G.ebt[lane] = g.ebt;
    G.ec[lane] = g.ec;
    if (lane == 0) G.fast = g.fast;
}

// One 32x32 score tile of chunk-local tokens, computed transposed:
// acc[s][t] = sum_key K[s][key] Q[t][key], s = 32J + row, t = 32I + column;
// lane l32 holds column t = 32I + perm5(l32) and element e row
// s = 32J + elem_index(0, e, h).  Masked (e^(g_t - g_s) where t >= s, else 0),
// packed to bf16 and stored into P (physical row 32I + l32).
// score_mask masks and stores a tile whose products are in acc.
__device__ __forceinline__ void score_mask(Smem& sm, const f32x16& acc, const Gates& G, int I, int J,
                                           int l32, int h) {
    const int qrow = 32 * I + l32;
    const int t = 32 * I + perm5(l32);
    auto mask = [&](auto weight, const float* ws, float et) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int s0 = 32 * J + elem_index(0, 4 * b, h);
            const f32x4 gs = *reinterpret_cast<const f32x4*>(&ws[s0]);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = weight(et, gs[i]) * acc[4 * b + i];
                p[i] = (I > J || t >= s0 + i) ? d : 0.f;
            }
            *reinterpret_cast<uint2*>(&sm.P[qrow * LT + s0]) = pack4(p[0], p[1], p[2], p[3]);
        }
    };
    if (__builtin_amdgcn_readfirstlane(G.fast))  // P'_ts = ec_t (q_t . k_s)
        mask([](float a, float) { return a; }, G.fl, G.ec[t]);
    else
        mask([](float a, float b) { return __builtin_amdgcn_exp2f(a - b); }, G.gl, G.gl[t]);
}
// Operands of score tile (I, J) at contraction step k (keys 16k + 8h ..).
__device__ __forceinline__ bf16x8 score_k(const uint16_t* Kb, int J, int k, int l32, int h) {
    return lds8(Kb + kidx(32 * J + l32, 16 * k + 8 * h));
}
__device__ __forceinline__ bf16x8 score_q(const Smem& sm, int I, int k, int l32, int h) {
    return lds8(&sm.Q[(32 * I + l32) * LQ + 16 * k + 8 * h]);
}
// Score tiles (1, 0) and (1, 1): one pass over their shared q rows, two
// independent MFMA chains interleaved, operands loaded two steps ahead.
__device__ __forceinline__ void score_tiles_row1(Smem& sm, const uint16_t* Kb, const Gates& G, int l32,
                                                 int h) {
    bf16x8 q[3], k0[3], k1[3];
    auto fetch = [&](int k) {
        q[k % 3] = score_q(sm, 1, k, l32, h);
        k0[k % 3] = score_k(Kb, 0, k, l32, h);
        k1[k % 3] = score_k(Kb, 1, k, l32, h);
    };
    fetch(0);
    fetch(1);
    f32x16 a0 = f32x16{}, a1 = f32x16{};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k + 2 < 8) fetch(k + 2);
        __builtin_amdgcn_sched_barrier(0);
        a0 = mfma32(k0[k % 3], q[k % 3], a0);
        a1 = mfma32(k1[k % 3], q[k % 3], a1);
    }
    score_mask(sm, a0, G, 1, 0, l32, h);
    score_mask(sm, a1, G, 1, 1, l32, h);
}

// Top (blk 0) or bottom (blk 1) diagonal 32x32 block of T = (I + A)^-1 from
// the transposed k-Gram tile At[blk]: its two 16x16 diagonal blocks by
// forward substitution (lane (sb, c) of the first 32 builds column c of
// block sb; lanes 32..63 repeat them), then T10 = -T11 A10 T00 on the fp32
// MFMA.  Written to D[blk].
__device__ __forceinline__ void solve_block(Smem& sm, int blk, int lane) {
    const float* At = sm.At[blk];
    float* Db = sm.D[blk];
    const int sb = (lane >> 4) & 1, cc = lane & 15;
    const float* Ab = At + 16 * sb * LS + 16 * sb;  // Ab[i * LS + r] = A[r][i] within the 16x16 block
    float x[16], acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    f32x4 row[3][4];  // rows i, i+1, i+2 of Ab in flight (4-entry groups from (i+1)/4 on)
    auto load_row = [&](int i, f32x4 (&dst)[4]) {
#pragma unroll
        for (int q = (i + 1) / 4; q < 4; ++q) dst[q] = *reinterpret_cast<const f32x4*>(&Ab[i * LS + 4 * q]);
    };
    load_row(0, row[0]);
    load_row(1, row[1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i + 2 < 16) load_row(i + 2, row[(i + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        const float xi = i == cc ? 1.f : -acc[i];
        x[i] = xi;
#pragma unroll
        for (int r = i + 1; r < 16; ++r) acc[r] = fmaf(row[i % 3][r >> 2][r & 3], xi, acc[r]);
    }
    if (lane < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Db[(16 * sb + r) * LS + 16 * sb + cc] = x[r];
    }
    lds_fence();
    // T10 = -T11 (A10 T00): lane (n16, g4) holds rows 4 g4 .. +3 of column n16
    const int n16 = lane & 15, g4 = lane >> 4;
    f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)  // A10[n16][4g4+kk] T00[4g4+kk][n16]
        y = mfma4(At[(4 * g4 + kk) * LS + 16 + n16], Db[(4 * g4 + kk) * LS + n16], y);
    const f32x4 at = *reinterpret_cast<const f32x4*>(&Db[(16 + n16) * LS + 16 + 4 * g4]);  // T11[n16][4g4+kk]
    f32x4 t10 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t10 = mfma4(at[kk], y[kk], t10);
#pragma unroll
    for (int r = 0; r < 4; ++r) Db[(16 + 4 * g4 + r) * LS + n16] = -t10[r];
}

// ----------------------------------------------------------------------------
// state waves (0, 1): chunk j's S-dependent products
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void state_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    constexpr bool OUT = ROLE != kLeafAggregate;  // o is read out (not for leaf aggregates)
    const int lane = threadIdx.x & 63, vb = wave_id();
    const int l32 = lane & 31, h = lane >> 5;
    // value channel of this lane within the slice, numbered through perm5 so
    // that the transposed read-out O^T (values as accumulator rows) holds 8
    // consecutive values per element group
    const int vl = 32 * vb + perm5(l32);
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
        const int unit = ROLE == kSequential || ROLE == kPrism ? un.head : un.head * job.leaves + un.leaf;
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
    // sbf[kk]: the state rounded to bf16 as B operands (contraction step kk)
    bf16x8 sbf[8];
    auto round_state = [&]() {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) sbf[kk] = sop(sacc, kk);
    };
    round_state();


    f32x16 qacc[2], xacc[2], oacc[2];
    for (int j = un.nb - 2; j < un.ne; ++j) {
        if (erows_done<ROLE>(sm, un, j)) break;
        const bool act = j >= un.nb;
        const uint16_t* Kb = sm.K[j & 1];
        // ---- first half: X = K S^T and O^T = S Q^T, four independent chains;
        // then the U-independent scalings of the second half ----
        if (act) {
            round_state();  // the state entering chunk j (updated in the previous step)
            // operands of contraction step k (keys 16k + 8h ..): k rows and q rows of
            // token tiles 0 and 1, loaded two steps ahead
            auto ka = [&](int k, int tt) { return lds8(Kb + kidx(32 * tt + l32, 16 * k + 8 * h)); };
            auto qb = [&](int k, int tt) { return lds8(&sm.Q[(32 * tt + l32) * LQ + 16 * k + 8 * h]); };
            bf16x8 kr[3][2], qr[3][2];
            auto fetch = [&](int k) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    if (GDN) kr[k % 3][tt] = ka(k, tt);
                    if (OUT) qr[k % 3][tt] = qb(k, tt);
                }
            };
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                xacc[tt] = f32x16{};
                qacc[tt] = f32x16{};
            }
            fetch(0);
            fetch(1);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (k + 2 < 8) fetch(k + 2);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    if (GDN) xacc[tt] = mfma32(kr[k % 3][tt], sbf[k], xacc[tt]);
                    if (OUT) qacc[tt] = mfma32(sbf[k], qr[k % 3][tt], qacc[tt]);
                }
            }
            // gamma_C S^T, and the gamma scaling of the read-out (column l32 of tile tt
            // is token t = 32 tt + perm5(l32): one gate per lane); the gates of chunk
            // j were formed two steps ago
            const Gates& G = sm.gate[j % 3];
            const float gC = G.gam[C - 1];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) sacc[jt] *= gC;
            if (OUT) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) oacc[tt] = qacc[tt] * G.gam[32 * tt + perm5(l32)];
            }
        }
        lds_barrier();
        // ---- second half: U, O (staged for the load waves), the state update ----
        if (act) {
            const Gates& G = sm.gate[j % 3];
            const uint16_t* Vb = sm.V[j & 1];
            const bool fast = __builtin_amdgcn_readfirstlane(G.fast);
            f32x16 uacc[2];
            if (GDN) {
                // U by block forward substitution over the two 32-token halves:
                // U_top = Tb_00 V_top + Tbn_00 X_top and
                // U_bot = Tb_11 V_bot + Tbn_11 X_bot + G U_top, with the diagonal blocks'
                // factors and G = -D_bot A_bl (conjugated by the decays on fast chunks)
                // from LDS (two accumulators per half halve the dependent chains)
                f32x16 va[2] = {f32x16{}, f32x16{}}, xa[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int t = kk >> 1;  // token half of this contraction step
                    const bf16x8 xo = sop(xacc, kk);
                    if (!un.erows) {  // rows of E: v = 0
                        const bf16x8 vo = v_operand(Vb, kk, 32 * vb, lane);
                        va[t] = mfma32(lds8(&sm.Tb[(32 * t + l32) * LT + 16 * kk + 8 * h]), vo, va[t]);
                    }
                    xa[t] = mfma32(lds8(&sm.Tbn[(32 * t + l32) * LT + 16 * kk + 8 * h]), xo, xa[t]);
                }
                uacc[0] = va[0] + xa[0];
                f32x16 ub = va[1] + xa[1];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    ub = mfma32(lds8(&sm.Tb[(32 + l32) * LT + 16 * ks + 8 * h]), sop(uacc, ks), ub);
                uacc[1] = ub;
            } else {
                // U = V; on fast chunks U' = diag(dec) V
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const bf16x8 v8 = v_operand(Vb, 2 * tt + s2, 32 * vb, lane);
                        const f32x8 d = fast ? ld8f(&G.dec[32 * tt + 16 * s2 + 8 * h]) : f32x8{1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
                        for (int i = 0; i < 8; ++i) uacc[tt][8 * s2 + i] = static_cast<float>(v8[i]) * d[i];
                    }
            }
            // U (U' on fast chunks) as bf16 operands: read-out and, on fast chunks, the
            // state update
            bf16x8 uo[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) uo[ks] = sop(uacc, ks);
            if (OUT) {
                // O^T = S Q^T diag(gamma) + U^T P^T
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    oacc[1] = mfma32(uo[ks], lds8(&sm.P[(32 + l32) * LT + 16 * ks + 8 * h]), oacc[1]);
                    if (ks < 2) oacc[0] = mfma32(uo[ks], lds8(&sm.P[l32 * LT + 16 * ks + 8 * h]), oacc[0]);
                }
                // element e holds value 32 vb + elem_index(0, e, h): elements 8s .. 8s+7 are
                // 8 consecutive values, one 16-byte LDS write each
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    uint16_t* orow = &sm.Ost[(32 * tt + perm5(l32)) * LO + 32 * vb + 8 * h];
                    *reinterpret_cast<bf16x8*>(orow) = half8<0>(oacc[tt]);
                    *reinterpret_cast<bf16x8*>(orow + 16) = half8<8>(oacc[tt]);
                }
            }
            // S^T <- gamma_C S^T + K^T diag(dec) U
            bf16x8 db[4];
            if (fast) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) db[ks] = uo[ks];
            } else {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const f32x8 d = ld8f(&G.dec[16 * ks + 8 * h]);
                    const f32x16& u = uacc[ks >> 1];
                    const int off = 8 * (ks & 1);
                    f32x8 x;
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = u[off + i] * d[i];
                    db[ks] = __builtin_convertvector(x, bf16x8);
                }
            }
            bf16x8 ko[2][4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) ko[0][jt] = kt_operand(Kb, 0, jt, lane);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k + 1 < 4) {
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) ko[(k + 1) & 1][jt] = kt_operand(Kb, k + 1, jt, lane);
                }
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) sacc[jt] = mfma32(ko[k & 1][jt], db[k], sacc[jt]);
            }
            if (ROLE == kLeafAggregate && un.erows) {  // rows of E: is the state exactly zero?
                bool nz = false;
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) nz |= sacc[jt][e] != 0.f;
                const bool any = __builtin_amdgcn_ballot_w64(nz) != 0;
                if (lane == 0) sm.ezero[vb] = any ? 0 : 1;
            }
        }
        lds_barrier();
    }

    float* dst = nullptr;
    if ((ROLE == kSequential || ROLE == kPrism) && job.S_out) dst = job.S_out + ((size_t)un.head * DV + vcol) * DK;
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
// load waves (4, 5): stage chunk j+1 and load chunk j+2; Tb, Tbn of T's
// diagonal block w - 4 of chunk j
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void load_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    constexpr bool OUT = ROLE != kLeafAggregate;  // q needed only where o is read out
    const int tid = threadIdx.x, lane = tid & 63, blk = wave_id() - 4;
    const int x = tid - 256;  // 0..127
    const int T = job.T;
    const size_t qk_base = (size_t)un.head * T * DK;
    const size_t v_base = (size_t)un.head * T * DV + un.r0;
    // q, k: keys 8jc..8jc+7 of tokens 32(i>>2) + 4tg + (i&3), i < 8;
    // v: values 8vc..8vc+7 of tokens 4vt + i, i < 4
    const int jc = x & 15, tg = x >> 4;
    const int vc = x & 7, vt = x >> 3;
    // (with the delta rule, k-Gram wave 3 stages the k rows: it holds them in
    // registers for its own products)
    uint4 qr[8], kr[8], vr[4];
    uint4 vr2[4];  // kPrism: the factor-row parts, merged at staging
    auto load = [&](int c) {
        if constexpr (ROLE == kPrism) {
            const PrismSrc P(job, un.head, un.r0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = c * C + 32 * (i >> 2) + 4 * tg + (i & 3);
                qr[i] = P.ld(P.q, P.q_rows(e) + 16 * jc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                unsigned a, b;
                P.rows(c * C + 4 * vt + i, DV, a, b);
                vr[i] = P.ld(P.v, a + 16 * vc);
                vr2[i] = P.ld(P.vf, b + 16 * vc);
            }
            return;
        }
        const Rows rq(job.q + qk_base, c, T, DK), rk(job.k + qk_base, c, T, DK), rv(job.v + v_base, c, T, DV);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 32 * (i >> 2) + 4 * tg + (i & 3);
            if (!GDN) kr[i] = rk.at(row, 8 * jc);
            if (OUT) qr[i] = rq.at(row, 8 * jc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = rv.at(4 * vt + i, 8 * vc);
    };
    auto stage = [&](int c) {
        uint16_t* Kb = sm.K[c & 1];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int prow = perm5(32 * (i >> 2) + 4 * tg + (i & 3));
            if (!GDN) *reinterpret_cast<uint4*>(Kb + kidx(prow, 8 * jc)) = kr[i];
            if (OUT) *reinterpret_cast<uint4*>(&sm.Q[prow * LQ + 8 * jc]) = qr[i];
        }
        uint16_t* Vb = sm.V[c & 1];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(&Vb[(4 * vt + i) * LV + 8 * vc]) = ROLE == kPrism ? orv(vr[i], vr2[i]) : vr[i];
    };
    // o of chunk c from the staged tile: 64 rows of 64 values (128 bytes), 8
    // rows of 8 16-byte pieces per store instruction; rows past T fall outside
    // the resource and are dropped
    auto store_o = [&](int c) {
        if (!job.o) return;
        if constexpr (ROLE == kPrism) {  // the token's last element only, as o_t
            const PrismSrc P(job, un.head, un.r0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int g = x + 128 * i, row = g >> 3, col = 8 * (g & 7);
                P.store_o(c * C + row, col, *reinterpret_cast<const uint4*>(&sm.Ost[row * LO + col]));
            }
            return;
        }
        const int valid = __builtin_amdgcn_readfirstlane(min(T - c * C, C));
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            job.o + ((size_t)un.head * T + (size_t)c * C) * DV + un.r0, (short)0,
            valid * DV * 2 - un.r0 * 2, 0x00020000);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = x + 128 * i, row = g >> 3, col = 8 * (g & 7);
            const uint4 w = *reinterpret_cast<const uint4*>(&sm.Ost[row * LO + col]);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, w), orsrc,
                (row * DV + col) * 2, 0, 0);
        }
    };
    // Tb = T diag(bw), Tbn = -T diag(beta gamma) over T's diagonal block blk:
    // lane (t, hh) converts row t, columns 16 hh .. 16 hh + 15 of the block
    auto convert = [&](int c) {
        const Gates& G = sm.gate[c % 3];
        const int t = lane & 31, hh = lane >> 5;
        const float* dr = sm.D[blk] + t * LS + 16 * hh;
        const int prow = 32 * blk + perm5(t);
        // row t scaled by dec_t on fast chunks (U' = diag(dec) U)
        const float rs = __builtin_amdgcn_readfirstlane(G.fast) ? G.dec[32 * blk + t] : 1.f;
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int s0 = 32 * blk + 16 * hh + 8 * q2;
            const f32x8 d = ld8f(dr + 8 * q2) * rs, w = ld8f(&G.bw[s0]), g = ld8f(&G.bg[s0]);
            *reinterpret_cast<uint4*>(&sm.Tb[prow * LT + s0]) = pack8(d * w);
            *reinterpret_cast<uint4*>(&sm.Tbn[prow * LT + s0]) = pack8(-(d * g));
        }
    };
    for (int j = un.nb - 2; j < un.ne; ++j) {
        if (erows_done<ROLE>(sm, un, j)) break;
        if (OUT && j - 1 >= un.nb) store_o(j - 1);
        if (GDN && j >= un.nb) convert(j);
        lds_barrier();
        if (j + 1 >= un.nb && j + 1 < un.ne) stage(j + 1);
        // the next chunk's rows overwrite the registers just staged: keep the
        // loads after the LDS writes (hoisted above them they would need a
        // second register set)
        __builtin_amdgcn_sched_barrier(0);
        if (j + 2 < un.ne) load(j + 2);
        lds_barrier();
    }
    if (OUT && un.ne - 1 >= un.nb) store_o(un.ne - 1);
}

// ----------------------------------------------------------------------------
// k-Gram waves (2, 3): chunk j+1's k-Gram tiles (wave 2 the diagonal ones in
// the first half, wave 3 the off-diagonal one in the second); wave 3 also chunk
// j's score tile (0,0), wave 2 the gates of chunk j+2
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void gram_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    constexpr bool OUT = ROLE != kLeafAggregate;
    const int lane = threadIdx.x & 63, blk = wave_id() - 2;
    const int l32 = lane & 31, h = lane >> 5;
    const int T = job.T;
    const size_t qk_base = (size_t)un.head * T * DK;
    // chunk c's k rows as MFMA operands, kreg[b][kk] = k[32b + l32][16kk + 8h .. +7],
    // loaded a chunk ahead of their use
    bf16x8 kreg[1][2][8];
    uint4 kreg2[2][8];  // kPrism: the factor-row parts, merged before the products
    auto load = [&](int c) {
        constexpr int st = 0;
        if constexpr (ROLE == kPrism) {
            const PrismSrc P(job, un.head, 0);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                unsigned oa, ob;
                P.rows(c * C + 32 * b + l32, DK, oa, ob);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    kreg[st][b][kk] = __builtin_bit_cast(bf16x8, P.ld(P.k, oa + 32 * kk + 16 * h));
                    kreg2[b][kk] = P.ld(P.kf, ob + 32 * kk + 16 * h);
                }
            }
            return;
        }
        const Rows rk(job.k + qk_base, c, T, DK);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                kreg[st][b][kk] = __builtin_bit_cast(bf16x8, rk.at(32 * b + l32, 16 * kk + 8 * h));
    };

    // kPrism: fold the factor-row parts in where the rows are first used
    auto merge = [&]() {
        if constexpr (ROLE == kPrism) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    kreg[0][b][kk] = __builtin_bit_cast(
                        bf16x8, orv(__builtin_bit_cast(uint4, kreg[0][b][kk]), kreg2[b][kk]));
        }
    };

    // k-Gram tile (I, J) masked into A, stored transposed: lane l32 holds
    // column s = 32J + l32, element e row t = 32I + 8(e>>2) + 4h + (e&3);
    // A_ts = exp2(gb_t - gl_s) (k_t . k_s) for t > s
    // (fast chunks: the weight is wt_t ws_s with ws = fl, wt = ebt; else
    // exp2(wt_t - ws_s) with ws = gl, wt = gb; w_s and w_t[b] = wt[32I + 8b + 4h ..]
    // are read before the products)
    auto gram_mask = [&](const f32x16& acc, int I, int J, bool fast, float w_s, const f32x4 (&w_t)[4],
                         float* dst) {
        const int s = 32 * J + l32;
        auto mask = [&](auto weight) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int t0 = 32 * I + 8 * b + 4 * h;
                f32x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d = weight(w_t[b][i], w_s) * acc[4 * b + i];
                    a[i] = (I > J || t0 + i > s) ? d : 0.f;
                }
                *reinterpret_cast<f32x4*>(&dst[l32 * LS + 8 * b + 4 * h]) = a;
            }
        };
        if (fast)
            mask([](float a, float b) { return a * b; });
        else
            mask([](float a, float b) { return __builtin_amdgcn_exp2f(a - b); });
    };

    // Wave 2 forms the gates two chunks ahead (second half, where it has no
    // other work), from alpha, beta, bw of token `lane`.  Their loads are issued
    // before the k rows of the next step, so the wait for them lets those rows
    // stay in flight.
    const size_t a_base = (size_t)un.head * T;
    const bool split = ROLE == kPrism || job.beta_w != job.beta;  // separate write strengths
    float pa = 1.f, pb = 0.f, pw = 0.f;
    float pl = 0.f;  // kPrism: the beta_l part of the write strength
    auto load_ab = [&](int c) {
        if constexpr (ROLE == kPrism) {
            PrismSrc(job, un.head, 0).gate_loads(c * C + lane, pa, pb, pl);
            return;
        }
        pa = ldtok(job.alpha + a_base, c, lane, T);
        if (GDN) {
            pb = ldtok(job.beta + a_base, c, lane, T);
            if (split) pw = ldtok(job.beta_w + a_base, c, lane, T);
        }
    };
    if (blk == 0 && un.nb < un.ne) load_ab(un.nb);

    // the two waves' loops compiled apart: with the waves' branches in one loop,
    // the compiler's memory-wait analysis merges their paths, and wave 2's wait
    // for its gate loads would also wait for the k rows it has just requested
    auto run = [&](auto blk_c) {
        constexpr int B = decltype(blk_c)::value;
        for (int j = un.nb - 2; j < un.ne; ++j) {
            if (erows_done<ROLE>(sm, un, j)) break;
            constexpr int st = 0;
            const int c = j + 1;  // chunk whose k-Gram tiles are built
            const bool build = GDN && c >= un.nb && c < un.ne;
            // mask weights of chunk c (its gates were formed two steps ago)
            auto weights = [&](bool& fast, const float*& ws, const float*& wt) {
                const Gates& G = sm.gate[c % 3];
                fast = __builtin_amdgcn_readfirstlane(G.fast);
                ws = fast ? G.fl : G.gl;
                wt = fast ? G.ebt : G.gb;
            };
            // ---- first half: wave 2 the diagonal k-Gram tiles of chunk c (the solve
            // reads them in the second half); wave 3 score tile (0,0) of chunk j ----
            if constexpr (B == 0) {
                if (build) {
                    merge();
                    bool fast;
                    const float *ws, *wt;
                    weights(fast, ws, wt);
                    f32x4 wt0[4], wt1[4];
    #pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        wt0[b] = *reinterpret_cast<const f32x4*>(&wt[8 * b + 4 * h]);
                        wt1[b] = *reinterpret_cast<const f32x4*>(&wt[32 + 8 * b + 4 * h]);
                    }
                    const float ws0 = ws[l32], ws1 = ws[32 + l32];
                    f32x16 a0 = f32x16{}, a1 = f32x16{};
    #pragma unroll
                    for (int kk = 0; kk < 8; ++kk) {
                        a0 = mfma32(kreg[st][0][kk], kreg[st][0][kk], a0);
                        a1 = mfma32(kreg[st][1][kk], kreg[st][1][kk], a1);
                    }
                    gram_mask(a0, 0, 0, fast, ws0, wt0, sm.At[0]);
                    gram_mask(a1, 1, 1, fast, ws1, wt1, sm.At[1]);
                }
                // chunk c + 1 goes into the registers just used: keep the loads after
                // their last use (hoisted above it they would need a second set).
                // Unconditional (chunks past the end read as zeros, with no memory
                // access): loads skipped on one path would make the wait for the
                // gate loads in the second half a wait for everything.
                __builtin_amdgcn_sched_barrier(0);
                if (GDN) load(c + 1);
            } else if (OUT && j >= un.nb) {
                const f32x16 sc = mfma_chain2<8>([&](int k) { return score_k(sm.K[j & 1], 0, k, l32, h); },
                                                 [&](int k) { return score_q(sm, 0, k, l32, h); }, f32x16{});
                score_mask(sm, sc, sm.gate[j % 3], 0, 0, l32, h);
            }
            lds_barrier();
            // ---- second half: wave 3 the off-diagonal k-Gram tile of chunk c into slot
            // c % 2 (wave 6 reads it in the next step), then chunk c + 1's rows ----
            if constexpr (B == 1) {
                if (build) {
                    merge();
                    bool fast;
                    const float *ws, *wt;
                    weights(fast, ws, wt);
                    f32x4 wt1[4];
    #pragma unroll
                    for (int b = 0; b < 4; ++b) wt1[b] = *reinterpret_cast<const f32x4*>(&wt[32 + 8 * b + 4 * h]);
                    const float ws0 = ws[l32];
                    f32x16 a = f32x16{};
    #pragma unroll
                    for (int kk = 0; kk < 8; ++kk) a = mfma32(kreg[st][1][kk], kreg[st][0][kk], a);
                    gram_mask(a, 1, 0, fast, ws0, wt1, sm.Ablt[c & 1]);
                    // chunk c's k rows into LDS for the other waves (row 32 b + l32 at
                    // LDS row perm5 of it), before the registers take chunk c + 1
                    uint16_t* Kb = sm.K[c & 1];
#pragma unroll
                    for (int b = 0; b < 2; ++b)
#pragma unroll
                        for (int kk = 0; kk < 8; ++kk)
                            *reinterpret_cast<bf16x8*>(Kb + kidx(perm5(32 * b + l32), 16 * kk + 8 * h)) =
                                kreg[st][b][kk];
                }
                __builtin_amdgcn_sched_barrier(0);
                if (GDN && c + 1 < un.ne) load(c + 1);
            } else if (j + 2 < un.ne) {
                // gates of chunk j + 2 into slot (j + 2) % 3: it held chunk j - 1, which
                // no wave reads after the previous step
                if constexpr (ROLE == kPrism)  // the loads' parts, merged here where they are used
                    PrismSrc(job, un.head, 0).gates_of((j + 2) * C + lane, pa, pb, pl, pa, pb, pw);
                form_gates(sm.gate[(j + 2) % 3], j + 2, pa, pb, split ? pw : pb, T, lane);
                load_ab(j + 3);  // (past the end: zeros, no memory access)
            }
            lds_barrier();
        }
    };
    if (blk == 0)
        run(std::integral_constant<int, 0>{});
    else
        run(std::integral_constant<int, 1>{});
}

// ----------------------------------------------------------------------------
// wave 6: T's off-diagonal block of chunk j; wave 7: chunk j's score tiles
// (1,0) and (1,1); then the diagonal blocks of chunk j+1's T
// ----------------------------------------------------------------------------
template <int MODE, int ROLE>
__device__ __forceinline__ void aux_role(Smem& sm, const ChunkJob& job, const Unit& un) {
    constexpr bool GDN = MODE == 0;
    constexpr bool OUT = ROLE != kLeafAggregate;
    const int lane = threadIdx.x & 63, w = wave_id();
    const int l32 = lane & 31, h = lane >> 5;
    (void)job;
    if (w == 6) {
        // the block of D above its diagonal (16x16, rows 0..15 x columns 16..31)
        // is zero for every chunk
        for (int i = lane; i < 2 * 256; i += 64) {
            const int b = i >> 8, r = (i >> 4) & 15, cc = i & 15;
            sm.D[b][r * LS + 16 + cc] = 0.f;
        }
    }
    for (int j = un.nb - 2; j < un.ne; ++j) {
        if (erows_done<ROLE>(sm, un, j)) break;
        if (j >= un.nb) {
            const Gates& G = sm.gate[j % 3];
            if (GDN && w == 6) {
                // G = -D_bot A_bl (bottom tokens x top tokens), computed as
                // Z^T = A_bl^T D_bot^T in split bf16 (every LDS input read up front):
                // lane l32 ends with row 32 + l32 of G, elements 8s2 .. 8s2+7 its
                // columns 16 s2 + 8 h .. +7.  On fast chunks U_top and U_bot come
                // scaled by dec, so G is conjugated: G_ts dec_t / dec_s = G_ts dec_t ec_s.
                const float* Ab = sm.Ablt[j & 1];
                const float* Db = sm.D[1];
                const int pr = perm5(l32);
                f32x8 ab[2], db[2], ev[2];
                const bool fast = __builtin_amdgcn_readfirstlane(G.fast);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    ab[kk] = ld8f(&Ab[pr * LS + 16 * kk + 8 * h]);
                    db[kk] = ld8f(&Db[l32 * LS + 16 * kk + 8 * h]);
                    ev[kk] = fast ? ld8f(&G.ec[16 * kk + 8 * h]) : f32x8{1, 1, 1, 1, 1, 1, 1, 1};
                }
                const float rs = fast ? -G.dec[32 + l32] : -1.f;
                f32x16 z = f32x16{};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) z = mfma_split(ab[kk], db[kk], z);
                const int prow = 32 + perm5(l32);
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const f32x8 zs = s2 ? __builtin_shufflevector(z, z, 8, 9, 10, 11, 12, 13, 14, 15)
                                        : __builtin_shufflevector(z, z, 0, 1, 2, 3, 4, 5, 6, 7);
                    *reinterpret_cast<uint4*>(&sm.Tb[prow * LT + 16 * s2 + 8 * h]) = pack8(zs * ev[s2] * rs);
                }
            }
            if (OUT && w == 7) {
                score_tiles_row1(sm, sm.K[j & 1], G, l32, h);
            }
        }
        lds_barrier();
        // ---- second half: diagonal block w - 6 of chunk j+1's T ----
        if (GDN && j + 1 >= un.nb && j + 1 < un.ne) solve_block(sm, w - 6, lane);
        lds_barrier();
    }
}

template <int MODE, int ROLE>
__global__ __launch_bounds__(NT, 1) void chunk_mfma_kernel(const ChunkJob job) {
    __shared__ Smem sm;
    const Unit un = unit_of<MODE, ROLE>(job);
    const int w = wave_id();
    if (w < 2)
        state_role<MODE, ROLE>(sm, job, un);
    else if (w == 2 || w == 3)
        gram_role<MODE, ROLE>(sm, job, un);
    else if (w == 4 || w == 5)
        load_role<MODE, ROLE>(sm, job, un);
    else
        aux_role<MODE, ROLE>(sm, job, un);
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
    else if (role == kPrism)
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kPrism>), dim3(2 * units), block, 0, stream, job);
    else if (role == kLeafAggregate) {
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kLeafAggregate>), dim3((MODE == 0 ? 4 : 2) * units), block, 0,
                           stream, job);
    }
    else
        hipLaunchKernelGGL((chunk_mfma_kernel<MODE, kLeafOutput>), dim3(2 * units), block, 0, stream, job);
    return hipGetLastError();
}

hipError_t launch_chunk_job(int mode, int role, const ChunkJob& job, hipStream_t stream) {
    if (role == kPrism) return launch_role<0>(role, job, stream);  // gated delta rule only
    return mode == 0 ? launch_role<0>(role, job, stream) : launch_role<1>(role, job, stream);
}

// floor(e / G) = mulhi(e, m) with m = ceil(2^32 / G) while e (G m - 2^32) < 2^32
static unsigned prism_magic(int G) { return (unsigned)(((1ull << 32) + G - 1) / G); }

bool chunk_prism_supported(int T, int L) {
    if (L < 1 || L > 8) return false;
    const unsigned long long G = L + 1, E = (unsigned long long)T * G;
    // byte offsets into one head's factor rows stay below 2^31 (buffer offsets
    // are 32-bit; 2^31 marks an unused source)
    return E < (1ull << 31) && E * (G * prism_magic((int)G) - (1ull << 32)) < (1ull << 32) &&
           (unsigned long long)T * L * DK * 2 < (1ull << 31) && (unsigned long long)T * L * DV * 2 < (1ull << 31);
}

hipError_t launch_chunk_prism(int BH, int T, int L, const void* q, const void* k, const void* v,
                              const void* kf, const void* vf, const float* alpha, const float* beta,
                              const float* beta_l, const float* S0, void* o, float* ST,
                              hipStream_t stream) {
    ChunkJob job{};
    job.q = static_cast<const uint16_t*>(q);
    job.k = static_cast<const uint16_t*>(k);
    job.v = static_cast<const uint16_t*>(v);
    job.alpha = alpha;
    job.beta = beta;
    job.beta_w = beta;
    job.o = static_cast<uint16_t*>(o);
    job.S_in = S0;
    job.S_out = ST;
    job.heads = BH;
    job.T = T * (L + 1);  // elements
    job.nchunks = (job.T + C - 1) / C;
    job.leaves = 1;
    job.leaf_chunks = job.nchunks;
    job.last_leaf = 0;
    job.prism_L = L;
    job.prism_T = T;
    job.prism_magic = prism_magic(L + 1);
    job.kf = static_cast<const uint16_t*>(kf);
    job.vf = static_cast<const uint16_t*>(vf);
    job.beta_l = beta_l;
    return launch_chunk_job(0, kPrism, job, stream);
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
