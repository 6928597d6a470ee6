// prism.hip -- PRISM's rank-L write factors, expanded into a split-strength scan stream.
//
// "PRISM: Parallel Residual Iterative Sequence Model" (gist.science explainer,
// technical summary 2.1-2.2; PRISM article, banbantang.com, section 3(2)-(4)):
// the state update S_t = S_{t-1} A_t + B_t keeps the gated-delta forget A_t and
// writes B_t = beta_t v_t k_t^T + sum_{l<=L} beta_t^(l) delta_t^(l) (k_t^(l))^T
// with factors that depend on the input only:
//
//   u_t        = sum_{j<w} c_j * x_{t-j}        short causal depthwise convolution
//   r^(1)      = v_t - u_t                      (u_t stands in for S_{t-1} k_t)
//   k^(l)      = W_k^(l) u_t,   p^(l) = W_p^(l) u_t
//   delta^(l)  = GELU(p^(l) * r^(l)),   r^(l+1) = r^(l) - delta^(l)
//
// Because nothing on the right depends on S, the scan itself is unchanged: a
// token becomes G = L + 1 consecutive elements of a split-strength scan,
//
//   element tG        : alpha_t, erase beta_t, write beta_t, k_t, v_t
//   element tG + l    : alpha 1, erase 0, write beta_t^(l), k^(l), delta^(l)
//
// with q_t on element tG + L (q = 0 on the others), so that element's output is
// o_t.  These kernels write that stream; the scan kernels run it.
//
// Two kernels:
//   * prism_mfma_kernel (bfloat16, dk = dv = 128): 64 tokens per workgroup.
//     The anchor is computed in float32 and kept as u = u_hi + u_lo (two
//     bfloat16 parts, ~16 significant bits); each projection is two
//     v_mfma_f32_32x32x16_bf16 passes (u_hi W + u_lo W) with float32
//     accumulation, so the factors carry float32-level accuracy until they are
//     rounded to bfloat16 on output.  Four waves: wave w computes channels
//     32w .. 32w+31 of both 32-token tiles (measured faster than eight waves
//     of one tile each, which load every weight row twice); its weight rows are
//     read straight into B-operand registers (the weights stay in L2 across
//     workgroups), the next matrix's while the current one is in use.  Output
//     tiles are staged in LDS and stored as whole 256-byte rows.  The
//     pass-through part of the stream is a separate streaming kernel.
//   * prism_plain_kernel (float32 or bfloat16, any supported size): the same
//     arithmetic with float32 FMAs, 16 tokens per workgroup.
#include <type_traits>

#include "common.hpp"
#include "gdscan.h"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, with erf from the rational
// approximation of Abramowitz and Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (after Hastings): for z >= 0,
//   erf z = 1 - (a1 s + a2 s^2 + a3 s^3 + a4 s^4 + a5 s^5) exp(-z^2),
//   s = 1 / (1 + p z),
// with absolute error at most 1.5e-7.  Branch-free (a library erff branches on
// |z| < 1, so a wave with both kinds of argument runs both paths).  With
// h = x (1 - erf z) / 2, z = |x| / sqrt 2, GELU is x - h for x >= 0 and h for
// x < 0 (no cancellation in the negative tail).
__device__ __forceinline__ float gelu(float x) {
    constexpr float p = 0.3275911f * 0.7071067811865476f;  // p / sqrt 2: s from |x|
    // a1 .. a5 halved: the polynomial gives (1 - erf z) / (2 exp(-z^2))
    constexpr float b1 = 0.5f * 0.254829592f, b2 = 0.5f * -0.284496736f, b3 = 0.5f * 1.421413741f,
                    b4 = 0.5f * -1.453152027f, b5 = 0.5f * 1.061405429f;
    const float sv = __builtin_amdgcn_rcpf(__builtin_fmaf(p, __builtin_fabsf(x), 1.f));
    const float poly = sv * __builtin_fmaf(sv, __builtin_fmaf(sv, __builtin_fmaf(sv, __builtin_fmaf(sv, b5, b4), b3), b2), b1);
    // exp(-z^2) = 2^(-x^2 log2(e) / 2)
    const float e = __builtin_amdgcn_exp2f(x * -0.7213475204444817f * x);
    const float h = x * poly * e;
    return x >= 0.f ? x - h : h;
}
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
// two floats rounded to bfloat16 (nearest even) in one register, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// 16-byte vector copies of the pass-through part of the stream (rows tG of k and
// v, every row of q, the gates) for tokens [t0, t0 + n) of head bh.
template <typename E>
__device__ __forceinline__ void copy_stream(const PrismJob& j, int bh, int t0, int n) {
    constexpr int V = 16 / sizeof(E);  // elements per 16-byte vector
    const int G = j.L + 1;
    const int tid = threadIdx.x;
    const size_t T2 = (size_t)j.T * G;
    const E* q = static_cast<const E*>(j.q);
    const E* k = static_cast<const E*>(j.k);
    const E* v = static_cast<const E*>(j.v);
    E* q2 = static_cast<E*>(j.q2);
    E* k2 = static_cast<E*>(j.k2);
    E* v2 = static_cast<E*>(j.v2);
    const int qv = j.dk / V, vv = j.dv / V;
    // q: rows tG .. tG + L, q_t on the last one
    for (int x = tid; x < n * G * qv; x += kThreads) {
        const int t = x / (G * qv), rem = x - t * (G * qv);
        const int g = rem / qv, c = rem - g * qv;
        const size_t tok = (size_t)bh * j.T + t0 + t;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (g == j.L) val = *reinterpret_cast<const uint4*>(q + tok * j.dk + c * V);
        *reinterpret_cast<uint4*>(q2 + ((size_t)bh * T2 + (size_t)(t0 + t) * G + g) * j.dk + c * V) = val;
    }
    for (int x = tid; x < n * qv; x += kThreads) {
        const int t = x / qv, c = x - t * qv;
        const size_t tok = (size_t)bh * j.T + t0 + t;
        *reinterpret_cast<uint4*>(k2 + ((size_t)bh * T2 + (size_t)(t0 + t) * G) * j.dk + c * V) =
            *reinterpret_cast<const uint4*>(k + tok * j.dk + c * V);
    }
    for (int x = tid; x < n * vv; x += kThreads) {
        const int t = x / vv, c = x - t * vv;
        const size_t tok = (size_t)bh * j.T + t0 + t;
        *reinterpret_cast<uint4*>(v2 + ((size_t)bh * T2 + (size_t)(t0 + t) * G) * j.dv + c * V) =
            *reinterpret_cast<const uint4*>(v + tok * j.dv + c * V);
    }
    // gates: alpha (alpha_t, 1, ...), erase (beta_t, 0, ...), write (beta_t, beta^(1), ...)
    float* be2 = j.beta2;
    float* bw2 = j.beta2 + (size_t)j.BH * T2;
    for (int x = tid; x < n * G; x += kThreads) {
        const int t = x / G, g = x - t * G;
        const size_t tok = (size_t)bh * j.T + t0 + t;
        const size_t e = (size_t)bh * T2 + (size_t)(t0 + t) * G + g;
        const float b = j.beta[tok];
        j.alpha2[e] = g == 0 ? j.alpha[tok] : 1.f;
        be2[e] = g == 0 ? b : 0.f;
        bw2[e] = g == 0 ? b : j.beta_l[tok * j.L + g - 1];
    }
}

// The pass-through part as a streaming kernel of its own (no arithmetic, few
// registers: many workgroups per CU keep HBM busy), 64 tokens per workgroup.
constexpr int kCopyTokens = 64;
template <typename E>
__global__ __launch_bounds__(kThreads) void prism_copy_kernel(const PrismJob j) {
    const int tiles = (j.T + kCopyTokens - 1) / kCopyTokens;
    const int bh = blockIdx.x / tiles;
    const int t0 = (blockIdx.x - bh * tiles) * kCopyTokens;
    copy_stream<E>(j, bh, t0, min(kCopyTokens, j.T - t0));
}

// ---------------------------------------------------------------------------
// plain kernel: float32 arithmetic, 16 tokens per workgroup
// ---------------------------------------------------------------------------
constexpr int kPlainTokens = 16;
constexpr int kMaxD = 128;

template <typename E>
__global__ __launch_bounds__(kThreads) void prism_plain_kernel(const PrismJob j) {
    __shared__ float u[kPlainTokens][kMaxD];
    __shared__ float r[kPlainTokens][kMaxD];
    const int tiles = (j.T + kPlainTokens - 1) / kPlainTokens;
    const int bh = blockIdx.x / tiles;
    const int t0 = (blockIdx.x - bh * tiles) * kPlainTokens;
    const int n = min(kPlainTokens, j.T - t0);
    const int head = bh % j.H;
    const int tid = threadIdx.x;
    const int G = j.L + 1;
    const size_t T2 = (size_t)j.T * G;
    const E* x = static_cast<const E*>(j.x);
    const E* v = static_cast<const E*>(j.v);
    const E* Wk = static_cast<const E*>(j.Wk);
    const E* Wp = static_cast<const E*>(j.Wp);
    E* k2 = static_cast<E*>(j.k2);
    E* v2 = static_cast<E*>(j.v2);
    const float* conv = j.conv + (size_t)head * j.W * j.dv;

    // anchor u and first residual r = v - u
    for (int e = tid; e < n * j.dv; e += kThreads) {
        const int t = e / j.dv, c = e - t * j.dv;
        const int tok = t0 + t;
        float s = 0.f;
        for (int i = 0; i < j.W && i <= tok; ++i)
            s += conv[i * j.dv + c] * io<E>::load(x, ((size_t)bh * j.T + tok - i) * j.dv + c);
        u[t][c] = s;
        r[t][c] = io<E>::load(v, ((size_t)bh * j.T + tok) * j.dv + c) - s;
    }
    __syncthreads();
    for (int l = 0; l < j.L; ++l) {
        const E* wk = Wk + ((size_t)head * j.L + l) * j.dk * j.dv;
        const E* wp = Wp + ((size_t)head * j.L + l) * j.dv * j.dv;
        for (int e = tid; e < n * j.dk; e += kThreads) {
            const int t = e / j.dk, i = e - t * j.dk;
            float s = 0.f;
            for (int c = 0; c < j.dv; ++c) s += io<E>::load(wk, (size_t)i * j.dv + c) * u[t][c];
            io<E>::store(k2, ((size_t)bh * T2 + (size_t)(t0 + t) * G + l + 1) * j.dk + i, s);
        }
        // each (t, i) of r belongs to one thread for every l: no barrier needed
        for (int e = tid; e < n * j.dv; e += kThreads) {
            const int t = e / j.dv, i = e - t * j.dv;
            float p = 0.f;
            for (int c = 0; c < j.dv; ++c) p += io<E>::load(wp, (size_t)i * j.dv + c) * u[t][c];
            const float d = gelu(p * r[t][i]);
            r[t][i] -= d;
            io<E>::store(v2, ((size_t)bh * T2 + (size_t)(t0 + t) * G + l + 1) * j.dv + i, d);
        }
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel: bfloat16, dk = dv = 128, 64 tokens per workgroup
// ---------------------------------------------------------------------------
constexpr int kTok = 64;
constexpr int kD = 128;
constexpr int kMfmaThreads = 256;  // 4 waves: wave w computes channels 32w .. 32w+31
constexpr int kLdu = kD + 8;  // padded row stride of the anchor tiles (bf16 elements)

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Writes the computed rows only (elements tG + l, l >= 1; the pass-through part
// comes from prism_copy_kernel), or, for the in-place scan, the same rows as
// compact factor arrays kf, vf [BH, T, L, 128].
// The products are formed transposed, D[channel][token] = W u^T (the weight
// rows are the A operand): each lane then holds four consecutive channels of
// one token per accumulator group and writes them to the LDS output tile as one
// 8-byte piece; whole 256-byte rows then go out from there.  (Stored straight
// from the accumulators, each store instruction would cover 32 rows with 16
// bytes each, which the memory system merges poorly.)
__global__ __launch_bounds__(kMfmaThreads, 3) void prism_mfma_kernel(const PrismJob j) {
    __shared__ __align__(16) uint16_t lds[3 * kTok * kLdu];
    uint16_t* const Uh = lds;                   // u rounded to bfloat16      [token][channel]
    uint16_t* const Ul = lds + kTok * kLdu;     // u - u_hi rounded to bfloat16
    uint16_t* const Ob = lds + 2 * kTok * kLdu; // v, then each output tile   [token][channel]
    // the anchor's inputs, staged where Uh and Ul go afterwards: x rows
    // t0 - (W - 1) .. t0 + n - 1 (zero before the sequence start) and the taps
    uint16_t* const Xs = lds;                                                     // [kTok + W - 1][kLdu]
    float* const Cs = reinterpret_cast<float*>(lds + (kTok + PRISM_MAX_WINDOW - 1) * kLdu);  // [W][128]
    static_assert((kTok + PRISM_MAX_WINDOW - 1) * kLdu * 2 + PRISM_MAX_WINDOW * kD * 4 <= 2 * kTok * kLdu * 2,
                  "anchor inputs fit over Uh and Ul");
    const int tiles = (j.T + kTok - 1) / kTok;
    const int bh = blockIdx.x / tiles;
    const int t0 = (blockIdx.x - bh * tiles) * kTok;
    const int n = min(kTok, j.T - t0);
    const int head = bh % j.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = j.W;
    const int G = j.L + 1;
    const size_t T2 = (size_t)j.T * G;
    const uint16_t* x = static_cast<const uint16_t*>(j.x);
    const uint16_t* v = static_cast<const uint16_t*>(j.v);
    const float* conv = j.conv + (size_t)head * W * kD;
    const uint16_t* Wk = static_cast<const uint16_t*>(j.Wk) + (size_t)head * j.L * kD * kD;
    const uint16_t* Wp = static_cast<const uint16_t*>(j.Wp) + (size_t)head * j.L * kD * kD;
    const int l32 = lane & 31, hh = lane >> 5;

    // A operands of weight matrix W [128 out][128 in]: row 32 w + l32 (this
    // wave's output channels), inputs 16 k + 8 hh .. + 7
    auto load_w = [&](const uint16_t* Wm, bf16x8 (&a)[8]) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = *reinterpret_cast<const bf16x8*>(Wm + (size_t)(32 * w + l32) * kD + 16 * k + 8 * hh);
    };
    bf16x8 wcur[8], wnext[8];

    // ---- stage x rows and taps (16 bytes a thread and pass), v rows into registers ----
    {
        constexpr int kPasses = ((kTok + PRISM_MAX_WINDOW - 1) * 16 + kMfmaThreads - 1) / kMfmaThreads;
        const int xrows = n + W - 1;
        uint4 xr[kPasses];
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            const int idx = tid + kMfmaThreads * i, r = idx >> 4;
            const int tok = t0 - (W - 1) + r;
            xr[i] = r < xrows && tok >= 0
                        ? *reinterpret_cast<const uint4*>(x + ((size_t)bh * j.T + tok) * kD + 8 * (idx & 15))
                        : make_uint4(0, 0, 0, 0);
        }
        f32x4 cr = {};
        if (tid < W * (kD / 4)) cr = *reinterpret_cast<const f32x4*>(conv + 4 * tid);
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            const int idx = tid + kMfmaThreads * i, r = idx >> 4;
            // (rows past the tile's tokens are zero: the anchor of every row is defined)
            if (r < kTok + W - 1) *reinterpret_cast<uint4*>(&Xs[r * kLdu + 8 * (idx & 15)]) = xr[i];
        }
        if (tid < W * (kD / 4)) *reinterpret_cast<f32x4*>(&Cs[4 * tid]) = cr;
    }
    uint4 vrow[4];  // 16 bytes of row tid / 16 + 16 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        vrow[i] = r < n ? *reinterpret_cast<const uint4*>(v + ((size_t)bh * j.T + t0 + r) * kD + 8 * (tid & 15))
                        : make_uint4(0, 0, 0, 0);
    }
    load_w(Wk, wcur);  // first matrix in flight during the anchor
    __syncthreads();

    // ---- anchor: thread (token tid/4, channels 32 (tid%4) .. +31), float32 ----
    {
        const int t = tid >> 2, cb = 32 * (tid & 3);
        float acc[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] = 0.f;
        // tap i reads x row t - i, staged at t + W - 1 - i
#pragma unroll
        for (int i = 0; i < PRISM_MAX_WINDOW; ++i) {
            if (i < W) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c0 = cb + 8 * g;
                    const uint4 xv = *reinterpret_cast<const uint4*>(&Xs[(t + W - 1 - i) * kLdu + c0]);
                    const f32x4 c_lo = *reinterpret_cast<const f32x4*>(&Cs[i * kD + c0]);
                    const f32x4 c_hi = *reinterpret_cast<const f32x4*>(&Cs[i * kD + c0 + 4]);
                    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float a0 = __uint_as_float(xw[q] << 16);
                        const float a1 = __uint_as_float(xw[q] & 0xffff0000u);
                        const float t0c = q < 2 ? c_lo[2 * q] : c_hi[2 * q - 4];
                        const float t1c = q < 2 ? c_lo[2 * q + 1] : c_hi[2 * q - 3];
                        acc[8 * g + 2 * q] += t0c * a0;
                        acc[8 * g + 2 * q + 1] += t1c * a1;
                    }
                }
            }
        }
        __syncthreads();  // every read of the staged inputs done: Uh, Ul go over them
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = acc[8 * g + 2 * q], b = acc[8 * g + 2 * q + 1];
                ph[q] = pack_bf16x2(a, b);
                pl[q] = pack_bf16x2(a - __uint_as_float(ph[q] << 16), b - __uint_as_float(ph[q] & 0xffff0000u));
            }
            *reinterpret_cast<uint4*>(&Uh[t * kLdu + cb + 8 * g]) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
            *reinterpret_cast<uint4*>(&Ul[t * kLdu + cb + 8 * g]) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&Ob[((tid >> 4) + 16 * i) * kLdu + 8 * (tid & 15)]) = vrow[i];
    __syncthreads();

    // Accumulator element e of token tile tt: token 32 tt + l32, channel
    // ch(e) = 32 w + 8 (e >> 2) + 4 hh + (e & 3); group g = e >> 2 holds four
    // consecutive channels from cg(g).
    auto cg = [&](int g) { return 32 * w + 8 * g + 4 * hh; };
    // residual r = v - u in the accumulator layout
    float res[2][16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int o = (32 * tt + l32) * kLdu + cg(g);
        const uint2 uh = *reinterpret_cast<const uint2*>(&Uh[o]);
        const uint2 ul = *reinterpret_cast<const uint2*>(&Ul[o]);
        const uint2 vv = *reinterpret_cast<const uint2*>(&Ob[o]);
        const uint32_t h4[4] = {uh.x << 16, uh.x & 0xffff0000u, uh.y << 16, uh.y & 0xffff0000u};
        const uint32_t l4[4] = {ul.x << 16, ul.x & 0xffff0000u, ul.y << 16, ul.y & 0xffff0000u};
        const uint32_t v4[4] = {vv.x << 16, vv.x & 0xffff0000u, vv.y << 16, vv.y & 0xffff0000u};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            res[tt][4 * g + i] = __uint_as_float(v4[i]) - (__uint_as_float(h4[i]) + __uint_as_float(l4[i]));
    }
    // token tile tt of W u^T (u = u_hi + u_lo): B operands are u rows
    auto project = [&](const bf16x8 (&a)[8], int tt) {
        f32x16 acc = {};
        const uint16_t* uh = &Uh[(32 * tt + l32) * kLdu + 8 * hh];
        const uint16_t* ul = &Ul[(32 * tt + l32) * kLdu + 8 * hh];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            acc = mfma32(a[k], *reinterpret_cast<const bf16x8*>(uh + 16 * k), acc);
            acc = mfma32(a[k], *reinterpret_cast<const bf16x8*>(ul + 16 * k), acc);
        }
        return acc;
    };
    // Ob -> element rows tG + l + 1 of the tile's tokens (or, with compact
    // factor rows, rows t L + l), 16 bytes a thread
    const bool compact = j.kf != nullptr;
    auto store_rows = [&](uint16_t* dst, int l) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 4) + 16 * i;
            const size_t row = compact ? ((size_t)bh * j.T + t0 + r) * j.L + l
                                       : (size_t)bh * T2 + (size_t)(t0 + r) * G + l + 1;
            if (r < n)
                *reinterpret_cast<uint4*>(dst + row * kD + 8 * (tid & 15)) =
                    *reinterpret_cast<const uint4*>(&Ob[r * kLdu + 8 * (tid & 15)]);
        }
    };
    // one projection into Ob, then its rows out: factor l from the weights in
    // wcur; IS_P: the correction delta = GELU(p r), r -= delta, else the
    // direction k itself
    auto emit = [&](auto is_p, int l) {
        constexpr bool IS_P = decltype(is_p)::value;
        __syncthreads();  // Ob free (v read, or the previous rows stored)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const f32x16 acc = project(wcur, tt);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * g + i;
                    if constexpr (IS_P) {
                        y[i] = gelu(acc[e] * res[tt][e]);
                        res[tt][e] -= y[i];
                    } else {
                        y[i] = acc[e];
                    }
                }
                const uint2 pk = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                *reinterpret_cast<uint2*>(&Ob[(32 * tt + l32) * kLdu + cg(g)]) = pk;
            }
        }
        __syncthreads();
        store_rows(static_cast<uint16_t*>(compact ? (IS_P ? j.vf : j.kf) : (IS_P ? j.v2 : j.k2)), l);
    };
    // 2L projections in the order Wk[0], Wp[0], Wk[1], ...; the next matrix's
    // operands load while the current one is in use
    for (int l = 0; l < j.L; ++l) {
        // (keeps the u operand reads inside the loop: hoisted, the 32 of them
        // would take 128 registers)
        asm volatile("" ::: "memory");
        load_w(Wp + (size_t)l * kD * kD, wnext);
        emit(std::false_type{}, l);
#pragma unroll
        for (int k = 0; k < 8; ++k) wcur[k] = wnext[k];
        if (l + 1 < j.L) load_w(Wk + (size_t)(l + 1) * kD * kD, wnext);
        asm volatile("" ::: "memory");
        emit(std::true_type{}, l);
#pragma unroll
        for (int k = 0; k < 8; ++k) wcur[k] = wnext[k];
    }
}

}  // namespace

hipError_t launch_prism_factors(const PrismJob& j, hipStream_t stream) {
    const unsigned grid = (unsigned)((size_t)j.BH * ((j.T + kTok - 1) / kTok));
    hipLaunchKernelGGL(prism_mfma_kernel, dim3(grid), dim3(kMfmaThreads), 0, stream, j);
    return hipGetLastError();
}

bool prism_supported(int dtype, int dk, int dv) {
    (void)dtype;
    const bool dk_ok = dk == 16 || dk == 32 || dk == 64 || dk == 128;
    const bool dv_ok = dv == 16 || dv == 32 || dv == 64 || dv == 128;
    return dk_ok && dv_ok;
}

hipError_t launch_prism_expand(int dtype, const PrismJob& j, hipStream_t stream) {
    const unsigned cgrid = (unsigned)((size_t)j.BH * ((j.T + kCopyTokens - 1) / kCopyTokens));
    if (dtype == 0)
        hipLaunchKernelGGL(prism_copy_kernel<float>, dim3(cgrid), dim3(kThreads), 0, stream, j);
    else
        hipLaunchKernelGGL(prism_copy_kernel<uint16_t>, dim3(cgrid), dim3(kThreads), 0, stream, j);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || j.L == 0) return e;  // no corrections: the copy is the stream
    if (dtype == 1 && j.dk == kD && j.dv == kD) {
        const unsigned grid = (unsigned)((size_t)j.BH * ((j.T + kTok - 1) / kTok));
        hipLaunchKernelGGL(prism_mfma_kernel, dim3(grid), dim3(kMfmaThreads), 0, stream, j);
    } else {
        const unsigned grid = (unsigned)((size_t)j.BH * ((j.T + kPlainTokens - 1) / kPlainTokens));
        if (dtype == 0)
            hipLaunchKernelGGL(prism_plain_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, j);
        else
            hipLaunchKernelGGL(prism_plain_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, stream, j);
    }
    return hipGetLastError();
}

}  // namespace gds
