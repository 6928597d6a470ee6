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
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int kThreads = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float gelu(float x) {
    return 0.5f * x * (1.f + erff(x * 0.7071067811865476f));
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

// Writes the computed rows only (elements tG + l, l >= 1); the pass-through part
// comes from prism_copy_kernel.
// (at most 256 VGPRs; 152 in use: three workgroups per CU)
__global__ __launch_bounds__(kMfmaThreads, 2) void prism_mfma_kernel(const PrismJob j) {
    __shared__ uint16_t Uh[kTok * kLdu];  // u rounded to bfloat16      [token][channel]
    __shared__ uint16_t Ul[kTok * kLdu];  // u - u_hi rounded to bfloat16
    __shared__ uint16_t Ob[kTok * kLdu];  // v, then each output tile    [token][channel]
    const int tiles = (j.T + kTok - 1) / kTok;
    const int bh = blockIdx.x / tiles;
    const int t0 = (blockIdx.x - bh * tiles) * kTok;
    const int n = min(kTok, j.T - t0);
    const int head = bh % j.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = j.L + 1;
    const size_t T2 = (size_t)j.T * G;
    const uint16_t* x = static_cast<const uint16_t*>(j.x);
    const uint16_t* v = static_cast<const uint16_t*>(j.v);
    uint16_t* k2 = static_cast<uint16_t*>(j.k2);
    uint16_t* v2 = static_cast<uint16_t*>(j.v2);
    const float* conv = j.conv + (size_t)head * j.W * kD;
    const uint16_t* Wk = static_cast<const uint16_t*>(j.Wk) + (size_t)head * j.L * kD * kD;
    const uint16_t* Wp = static_cast<const uint16_t*>(j.Wp) + (size_t)head * j.L * kD * kD;
    const int l32 = lane & 31, hh = lane >> 5;
    const int nc = 32 * w + l32;

    // B operands of weight matrix W [128 out][128 in]: rows nc of this wave
    auto load_b = [&](const uint16_t* W, bf16x8 (&b)[8]) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            b[k] = *reinterpret_cast<const bf16x8*>(W + (size_t)nc * kD + 16 * k + 8 * hh);
    };
    bf16x8 bcur[8], bnext[8];
    load_b(Wk, bcur);  // first matrix in flight during the anchor

    // rows [t0, t0 + n) of a [T][128] bf16 tensor of head bh: thread tid moves
    // 16 bytes of row r = tid / 16 + 32 i
    auto tile_rows = [&](const uint16_t* src, uint4 (&dst)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 4) + 16 * i;
            dst[i] = r < n ? *reinterpret_cast<const uint4*>(src + ((size_t)bh * j.T + t0 + r) * kD + 8 * (tid & 15))
                           : make_uint4(0, 0, 0, 0);
        }
    };
    uint4 vrow[4];
    tile_rows(v, vrow);

    // ---- anchor: thread (token tid/8, channels 16 (tid%8) .. +15), float32 ----
    {
        const int t = tid >> 2, cb = 32 * (tid & 3);
        const int tok = t0 + t;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c0 = cb + 8 * g;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (t < n) {
                for (int i = 0; i < j.W && i <= tok; ++i) {
                    const uint4 xv = *reinterpret_cast<const uint4*>(x + ((size_t)bh * j.T + tok - i) * kD + c0);
                    const f32x4 c_lo = *reinterpret_cast<const f32x4*>(conv + i * kD + c0);
                    const f32x4 c_hi = *reinterpret_cast<const f32x4*>(conv + i * kD + c0 + 4);
                    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float a0 = __uint_as_float(xw[q] << 16);
                        const float a1 = __uint_as_float(xw[q] & 0xffff0000u);
                        const float t0c = q < 2 ? c_lo[2 * q] : c_hi[2 * q - 4];
                        const float t1c = q < 2 ? c_lo[2 * q + 1] : c_hi[2 * q - 3];
                        acc[2 * q] += t0c * a0;
                        acc[2 * q + 1] += t1c * a1;
                    }
                }
            }
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = f32_to_bf16(acc[e]);
                lo[e] = f32_to_bf16(acc[e] - bf16_to_f32(hi[e]));
            }
            uint4 ph, pl;
            ph.x = hi[0] | (uint32_t)hi[1] << 16; ph.y = hi[2] | (uint32_t)hi[3] << 16;
            ph.z = hi[4] | (uint32_t)hi[5] << 16; ph.w = hi[6] | (uint32_t)hi[7] << 16;
            pl.x = lo[0] | (uint32_t)lo[1] << 16; pl.y = lo[2] | (uint32_t)lo[3] << 16;
            pl.z = lo[4] | (uint32_t)lo[5] << 16; pl.w = lo[6] | (uint32_t)lo[7] << 16;
            *reinterpret_cast<uint4*>(&Uh[t * kLdu + c0]) = ph;
            *reinterpret_cast<uint4*>(&Ul[t * kLdu + c0]) = pl;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&Ob[((tid >> 4) + 16 * i) * kLdu + 8 * (tid & 15)]) = vrow[i];
    __syncthreads();

    // accumulator element e of token tile tt is token 32 tt + row(e), channel nc
    auto row = [&](int e) { return 8 * (e >> 2) + 4 * hh + (e & 3); };
    // residual r = v - u in the accumulator layout
    float res[2][16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int t = 32 * tt + row(e);
        const float uu = bf16_to_f32(Uh[t * kLdu + nc]) + bf16_to_f32(Ul[t * kLdu + nc]);
        res[tt][e] = bf16_to_f32(Ob[t * kLdu + nc]) - uu;
    }
    // token tile tt of u W^T (u = u_hi + u_lo)
    auto project = [&](const bf16x8 (&b)[8], int tt) {
        f32x16 a = {};
        const uint16_t* uh = &Uh[(32 * tt + l32) * kLdu + 8 * hh];
        const uint16_t* ul = &Ul[(32 * tt + l32) * kLdu + 8 * hh];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            a = mfma32(*reinterpret_cast<const bf16x8*>(uh + 16 * k), b[k], a);
            a = mfma32(*reinterpret_cast<const bf16x8*>(ul + 16 * k), b[k], a);
        }
        return a;
    };
    // Ob -> element rows tG + l + 1 of the tile's tokens, 16 bytes a thread
    auto store_rows = [&](uint16_t* dst, int l) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 4) + 16 * i;
            if (r < n)
                *reinterpret_cast<uint4*>(dst + ((size_t)bh * T2 + (size_t)(t0 + r) * G + l + 1) * kD + 8 * (tid & 15)) =
                    *reinterpret_cast<const uint4*>(&Ob[r * kLdu + 8 * (tid & 15)]);
        }
    };
    // 2L projections in the order Wk[0], Wp[0], Wk[1], ...; the next matrix's
    // operands load while the current one is in use
    for (int m = 0; m < 2 * j.L; ++m) {
        const int l = m >> 1;
        const bool is_p = m & 1;
        if (m + 1 < 2 * j.L) load_b(((m + 1) & 1 ? Wp : Wk) + (size_t)((m + 1) >> 1) * kD * kD, bnext);
        __syncthreads();  // Ob free (v read, or the previous rows stored)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const f32x16 acc = project(bcur, tt);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float y = acc[e];
                if (is_p) {  // delta = GELU(p r), r -= delta
                    y = gelu(acc[e] * res[tt][e]);
                    res[tt][e] -= y;
                }
                Ob[(32 * tt + row(e)) * kLdu + nc] = f32_to_bf16(y);
            }
        }
        __syncthreads();
        store_rows(is_p ? v2 : k2, l);
#pragma unroll
        for (int k = 0; k < 8; ++k) bcur[k] = bnext[k];
    }
}

}  // namespace

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
