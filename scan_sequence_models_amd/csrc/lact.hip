// lact.hip -- large-chunk fast-weight update with linear fast weights.
//
// "块级更新与端到端 TTT" (PaperTrace 5.2, opening section) and the LaCT news
// article (senqingzn.com, the large-chunk test-time-training layer and its
// update/apply paragraph): a fast weight W (d_v x d_k) per head is trained on
// the sequence with the key-value reconstruction loss |W k - v|^2 / 2, one
// gradient step per chunk of m tokens with every gradient of the chunk taken at
// the chunk's starting weight:
//
//   W_{b+1} = W_b - sum_{i in B_b} eta_i (W_b k_i - v_i) k_i^T
//           = W_b + F_b - W_b G_b,     G_b = K^T diag(eta) K,  F_b = V^T diag(eta) K
//
// and each query reads o_i = W q_i with W = W_{b+1} (update then apply: a
// token sees its whole chunk) or W = W_b (apply then update: the mask shifted
// by one chunk).  This is the affine scan at chunk granularity
// (E_b = I - G_b, f_b = F_b); G and F are large contractions over the chunk's
// tokens, so the work splits in three:
//
//   lact_stats_kernel  (all chunks in parallel)  G_b, F_b, split-bf16 MFMA
//   lact_recur_kernel  (per head, chunk by chunk) W_{b+1} = W_b + F_b - W_b G_b,
//                                                  float32 MFMA, W in LDS
//   lact_apply_kernel  (all tokens in parallel)   O = Q W_use^T, bf16 MFMA
//
// for bfloat16 data with d_k = d_v = 128 and m a multiple of 64, and
// lact_plain_kernel (one workgroup per head, float32 FMAs) for d <= 64.
#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// plain kernel: one workgroup per head, everything in LDS (d <= 64)
// ---------------------------------------------------------------------------
constexpr int kPlainD = 64;

template <typename E>
__global__ __launch_bounds__(kThreads) void lact_plain_kernel(const LactJob j) {
    __shared__ float W[kPlainD * kPlainD];   // [dv][dk]
    __shared__ float Wn[kPlainD * kPlainD];  // next weight
    __shared__ float G[kPlainD * kPlainD];   // [dk][dk]
    __shared__ float F[kPlainD * kPlainD];   // [dv][dk]
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int dk = j.dk, dv = j.dv, T = j.T;
    const E* q = static_cast<const E*>(j.q) + (size_t)bh * T * dk;
    const E* k = static_cast<const E*>(j.k) + (size_t)bh * T * dk;
    const E* v = static_cast<const E*>(j.v) + (size_t)bh * T * dv;
    const float* eta = j.eta + (size_t)bh * T;
    E* o = static_cast<E*>(j.o) + (size_t)bh * T * dv;
    for (int x = tid; x < dv * dk; x += kThreads) W[x] = j.W0 ? j.W0[(size_t)bh * dv * dk + x] : 0.f;
    for (int s = 0; s < T; s += j.chunk) {
        const int e = min(s + j.chunk, T);
        __syncthreads();
        for (int x = tid; x < dk * dk; x += kThreads) {
            const int a = x / dk, b = x - a * dk;
            float acc = 0.f;
            for (int t = s; t < e; ++t)
                acc += eta[t] * io<E>::load(k, (size_t)t * dk + a) * io<E>::load(k, (size_t)t * dk + b);
            G[x] = acc;
        }
        for (int x = tid; x < dv * dk; x += kThreads) {
            const int a = x / dk, b = x - a * dk;
            float acc = 0.f;
            for (int t = s; t < e; ++t)
                acc += eta[t] * io<E>::load(v, (size_t)t * dv + a) * io<E>::load(k, (size_t)t * dk + b);
            F[x] = acc;
        }
        __syncthreads();
        for (int x = tid; x < dv * dk; x += kThreads) {  // W + F - W G
            const int a = x / dk, b = x - a * dk;
            float acc = 0.f;
            for (int c = 0; c < dk; ++c) acc += W[a * dk + c] * G[c * dk + b];
            Wn[x] = W[x] + F[x] - acc;
        }
        __syncthreads();
        const float* Wu = j.order == 0 ? Wn : W;
        for (int x = tid; x < (e - s) * dv; x += kThreads) {
            const int t = s + x / dv, a = x - (x / dv) * dv;
            float acc = 0.f;
            for (int c = 0; c < dk; ++c) acc += Wu[a * dk + c] * io<E>::load(q, (size_t)t * dk + c);
            io<E>::store(o, (size_t)t * dv + a, acc);
        }
        __syncthreads();
        for (int x = tid; x < dv * dk; x += kThreads) W[x] = Wn[x];
    }
    __syncthreads();
    if (j.WT)
        for (int x = tid; x < dv * dk; x += kThreads) j.WT[(size_t)bh * dv * dk + x] = W[x];
}

// ---------------------------------------------------------------------------
// MFMA path (bf16, d = 128)
// ---------------------------------------------------------------------------
constexpr int kD = 128;
constexpr int kTok = 64;        // tokens per staged tile
constexpr int kLdt = kD + 32;   // row stride (bf16) of staged [token][channel] tiles:
                                // transpose reads of 4 rows x 16 columns are conflict-free

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand of a 32x32x16 MFMA contracted over the rows (tokens) of a row-major
// [token][channel] bf16 tile in LDS: lane (c = lane % 32, g = lane / 32) gets
// tokens row0 + 8 g .. +7 of channel col0 + c, by two ds_read_b64_tr_b16 (in
// each 16-lane group, lane l receives element l % 4 of the 8-byte pieces that
// lanes 4 i + l / 4 address, i = 0..3: four consecutive rows of one column).
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int row0, int col0, int lane) {
    const int l = lane & 15, grp = lane >> 4;
    const int r = row0 + 8 * (grp >> 1) + (l >> 2);
    const int c = col0 + 16 * (grp & 1) + 4 * (l & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + r * kLdt + c));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + (r + 4) * kLdt + c));
    const s16x4 ab[2] = {a, b};
    return __builtin_bit_cast(bf16x8, ab);
}

// eta * x split into two bf16 parts (hi + lo carries ~16 significant bits)
__device__ __forceinline__ void scale_split(bf16x8 x, const float (&e)[8], bf16x8& hi, bf16x8& lo) {
    f32x4 p0, p1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = static_cast<float>(x[i]) * e[i];
        p1[i] = static_cast<float>(x[4 + i]) * e[4 + i];
    }
    const bf16x4 h0 = __builtin_convertvector(p0, bf16x4), h1 = __builtin_convertvector(p1, bf16x4);
    f32x4 r0, r1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r0[i] = p0[i] - static_cast<float>(h0[i]);
        r1[i] = p1[i] - static_cast<float>(h1[i]);
    }
    const bf16x4 l0 = __builtin_convertvector(r0, bf16x4), l1 = __builtin_convertvector(r1, bf16x4);
    hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// G_b (and F_b) partial sums over one split of a chunk: workgroup (unit, chunk,
// split) of 4 waves; wave w owns rows 32w .. 32w+31 of G and F (four 32x32
// tiles each).  Tokens come in tiles of 64, double-buffered in LDS.
__global__ __launch_bounds__(kThreads, 1) void lact_stats_kernel(const LactJob j) {
    __shared__ uint16_t Ks[2][kTok * kLdt];
    __shared__ uint16_t Vs[2][kTok * kLdt];
    __shared__ float Es[2][kTok];
    const int nch = (j.T + j.chunk - 1) / j.chunk;
    const int x = blockIdx.x;
    const int split = x % j.nsplit, cb = (x / j.nsplit) % nch, bh = x / (j.nsplit * nch);
    const int t_begin = cb * j.chunk + split * j.split_tokens;
    const int t_end = min(min(t_begin + j.split_tokens, (cb + 1) * j.chunk), j.T);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint16_t* k = static_cast<const uint16_t*>(j.k) + (size_t)bh * j.T * kD;
    const uint16_t* v = static_cast<const uint16_t*>(j.v) + (size_t)bh * j.T * kD;
    const float* eta = j.eta + (size_t)bh * j.T;

    // prefetch of one tile: thread moves 16 bytes of rows tid/16 + 16 i of k and v
    uint4 kr[4], vr[4];
    float er = 0.f;
    auto fetch = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + (tid >> 4) + 16 * i;
            const bool in = t < t_end;
            kr[i] = in ? *reinterpret_cast<const uint4*>(k + (size_t)t * kD + 8 * (tid & 15)) : make_uint4(0, 0, 0, 0);
            vr[i] = in ? *reinterpret_cast<const uint4*>(v + (size_t)t * kD + 8 * (tid & 15)) : make_uint4(0, 0, 0, 0);
        }
        if (tid < kTok) er = t0 + tid < t_end ? eta[t0 + tid] : 0.f;  // pad rows: eta 0
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 4) + 16 * i;
            *reinterpret_cast<uint4*>(&Ks[buf][r * kLdt + 8 * (tid & 15)]) = kr[i];
            *reinterpret_cast<uint4*>(&Vs[buf][r * kLdt + 8 * (tid & 15)]) = vr[i];
        }
        if (tid < kTok) Es[buf][tid] = er;
    };

    f32x16 g[4], f[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) g[J] = f[J] = f32x16{};
    const int ntiles = (t_end - t_begin + kTok - 1) / kTok;
    if (ntiles > 0) {
        fetch(t_begin);
        stage(0);
    }
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntiles) fetch(t_begin + (it + 1) * kTok);
        __syncthreads();  // tile it staged; the other buffer is free
        const uint16_t* K = Ks[buf];
        const uint16_t* V = Vs[buf];
#pragma unroll
        for (int s = 0; s < kTok / 16; ++s) {
            // eta of this lane's eight tokens 16 s + 8 (lane / 32) + e
            float e8[8];
            const f32x4 ea = *reinterpret_cast<const f32x4*>(&Es[buf][16 * s + 8 * (lane >> 5)]);
            const f32x4 eb = *reinterpret_cast<const f32x4*>(&Es[buf][16 * s + 8 * (lane >> 5) + 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) { e8[i] = ea[i]; e8[4 + i] = eb[i]; }
            bf16x8 b[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) b[J] = tr_operand(K, 16 * s, 32 * J, lane);
            bf16x8 gh, gl, fh, fl;
            scale_split(b[w], e8, gh, gl);                        // rows 32w.. of eta K
            scale_split(tr_operand(V, 16 * s, 32 * w, lane), e8, fh, fl);  // rows of eta V
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                g[J] = mfma32(gh, b[J], g[J]);
                g[J] = mfma32(gl, b[J], g[J]);
                f[J] = mfma32(fh, b[J], f[J]);
                f[J] = mfma32(fl, b[J], f[J]);
            }
        }
        if (it + 1 < ntiles) stage(buf ^ 1);
    }
    // partials: slot (bh, cb, split), [G | F] each [128][128] row-major;
    // lane (n, h) holds rows 8 b + 4 h + r of column n of each tile
    float* out = j.ws_stats + ((size_t)(bh * nch + cb) * j.nsplit + split) * 2 * kD * kD;
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = 32 * w + 8 * (e >> 2) + 4 * h + (e & 3);
            out[row * kD + 32 * J + n] = g[J][e];
            out[kD * kD + row * kD + 32 * J + n] = f[J][e];
        }
}

// Chunk-by-chunk recursion of one head: W (fp32) in LDS; W G on the fp32 MFMA
// (16x16x4); each chunk's applied weight leaves as bf16 for the apply kernel.
constexpr int kLdw = kD + 4;  // fp32 row stride in LDS
__global__ __launch_bounds__(kThreads, 1) void lact_recur_kernel(const LactJob j) {
    __shared__ float Wl[kD * kLdw];  // W_b       [dv][dk]
    __shared__ float Gl[kD * kLdw];  // G_b       [dk][dk]
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = (j.T + j.chunk - 1) / j.chunk;
    for (int x = tid; x < kD * kD; x += kThreads)
        Wl[(x >> 7) * kLdw + (x & 127)] = j.W0 ? j.W0[(size_t)bh * kD * kD + x] : 0.f;
    // wave w: rows 32w .. 32w+31 of the product, as 2 x 8 blocks of 16x16;
    // lane (c = lane % 16, g = lane / 16) holds rows 4g .. 4g+3 of column c
    const int c16 = lane & 15, g4 = lane >> 4;
    auto store_bf16 = [&](uint16_t* dst) {  // Wl -> bf16 [dv][dk]
        for (int x = tid; x < kD * kD; x += kThreads)
            dst[x] = f32_to_bf16(Wl[(x >> 7) * kLdw + (x & 127)]);
    };
    for (int cb = 0; cb < nch; ++cb) {
        const float* st = j.ws_stats + (size_t)(bh * nch + cb) * j.nsplit * 2 * kD * kD;
        __syncthreads();  // previous W final in Wl
        for (int x = tid; x < kD * kD; x += kThreads) {
            float gsum = 0.f;
            for (int s = 0; s < j.nsplit; ++s) gsum += st[(size_t)s * 2 * kD * kD + x];
            Gl[(x >> 7) * kLdw + (x & 127)] = gsum;
        }
        if (j.order == 1) store_bf16(j.ws_wuse + (size_t)(bh * nch + cb) * kD * kD);
        __syncthreads();
        // new rows of W: W + F - W G, accumulated in registers
        f32x4 acc[2][8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cbk = 0; cbk < 8; ++cbk) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                const int r0 = 32 * w + 16 * rb;
                for (int kk = 0; kk < kD; kk += 4) {
                    const float av = Wl[(r0 + c16) * kLdw + kk + g4];  // A[m = c16][k = g4]
                    const float bv = Gl[(kk + g4) * kLdw + 16 * cbk + c16];  // B[k = g4][n = c16]
                    a = mfma4(av, bv, a);
                }
                acc[rb][cbk] = a;
            }
        __syncthreads();  // every read of the old W done
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cbk = 0; cbk < 8; ++cbk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 32 * w + 16 * rb + 4 * g4 + r, col = 16 * cbk + c16;
                    float fsum = 0.f;
                    for (int s = 0; s < j.nsplit; ++s)
                        fsum += st[(size_t)s * 2 * kD * kD + kD * kD + row * kD + col];
                    Wl[row * kLdw + col] += fsum - acc[rb][cbk][r];
                }
        __syncthreads();
        if (j.order == 0) store_bf16(j.ws_wuse + (size_t)(bh * nch + cb) * kD * kD);
    }
    __syncthreads();
    if (j.WT)
        for (int x = tid; x < kD * kD; x += kThreads) j.WT[(size_t)bh * kD * kD + x] = Wl[(x >> 7) * kLdw + (x & 127)];
}

// O = Q W_use^T for 64 tokens of one head: wave w computes channels 32w ..
// 32w+31 for both 32-token tiles; W rows go straight into B-operand registers;
// the output is staged in LDS and stored as whole 256-byte rows.
constexpr int kLdo = kD + 8;
__global__ __launch_bounds__(kThreads, 2) void lact_apply_kernel(const LactJob j) {
    __shared__ uint16_t Qs[kTok * kLdo];
    __shared__ uint16_t Os[kTok * kLdo];
    const int tiles = (j.T + kTok - 1) / kTok;
    const int bh = blockIdx.x / tiles;
    const int t0 = (blockIdx.x - bh * tiles) * kTok;
    const int n = min(kTok, j.T - t0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int nch = (j.T + j.chunk - 1) / j.chunk;
    const uint16_t* q = static_cast<const uint16_t*>(j.q) + (size_t)bh * j.T * kD;
    uint16_t* o = static_cast<uint16_t*>(j.o) + (size_t)bh * j.T * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        *reinterpret_cast<uint4*>(&Qs[r * kLdo + 8 * (tid & 15)]) =
            r < n ? *reinterpret_cast<const uint4*>(q + (size_t)(t0 + r) * kD + 8 * (tid & 15)) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    // the 64 tokens may span two chunks (chunk is a multiple of 64: they do not)
    const int cb = t0 / j.chunk;
    const uint16_t* Wu = j.ws_wuse + ((size_t)bh * nch + cb) * kD * kD;
    const int nc = 32 * w + l32;
    bf16x8 b[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) b[kk] = *reinterpret_cast<const bf16x8*>(Wu + (size_t)nc * kD + 16 * kk + 8 * hh);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        f32x16 acc = {};
        const uint16_t* qr = &Qs[(32 * tt + l32) * kLdo + 8 * hh];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) acc = mfma32(*reinterpret_cast<const bf16x8*>(qr + 16 * kk), b[kk], acc);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            Os[(32 * tt + 8 * (e >> 2) + 4 * hh + (e & 3)) * kLdo + nc] = f32_to_bf16(acc[e]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        if (r < n)
            *reinterpret_cast<uint4*>(o + (size_t)(t0 + r) * kD + 8 * (tid & 15)) =
                *reinterpret_cast<const uint4*>(&Os[r * kLdo + 8 * (tid & 15)]);
    }
}

}  // namespace

bool lact_mfma_supported(int dtype, int dk, int dv, int chunk) {
    return dtype == 1 && dk == kD && dv == kD && chunk >= kTok && chunk % kTok == 0;
}
bool lact_plain_supported(int dk, int dv) {
    return (dk == 16 || dk == 32 || dk == 64) && (dv == 16 || dv == 32 || dv == 64);
}
constexpr int kSplitTokens = 2048;
int lact_splits(int chunk) { return (chunk + kSplitTokens - 1) / kSplitTokens; }
size_t lact_workspace_bytes(int64_t heads, int T, int chunk) {
    const int64_t nch = (T + chunk - 1) / chunk;
    return (size_t)heads * nch * ((size_t)lact_splits(chunk) * 2 * kD * kD * 4 + (size_t)kD * kD * 2);
}

hipError_t launch_lact(int dtype, LactJob j, void* workspace, hipStream_t stream) {
    if (!lact_mfma_supported(dtype, j.dk, j.dv, j.chunk)) {
        if (dtype == 0)
            hipLaunchKernelGGL(lact_plain_kernel<float>, dim3(j.BH), dim3(kThreads), 0, stream, j);
        else
            hipLaunchKernelGGL(lact_plain_kernel<uint16_t>, dim3(j.BH), dim3(kThreads), 0, stream, j);
        return hipGetLastError();
    }
    const int nch = (j.T + j.chunk - 1) / j.chunk;
    j.nsplit = lact_splits(j.chunk);
    j.split_tokens = (j.chunk + j.nsplit - 1) / j.nsplit;
    j.split_tokens = (j.split_tokens + kTok - 1) / kTok * kTok;
    j.ws_stats = static_cast<float*>(workspace);
    j.ws_wuse = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                            (size_t)j.BH * nch * j.nsplit * 2 * kD * kD * 4);
    hipLaunchKernelGGL(lact_stats_kernel, dim3((unsigned)((size_t)j.BH * nch * j.nsplit)), dim3(kThreads), 0,
                       stream, j);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lact_recur_kernel, dim3(j.BH), dim3(kThreads), 0, stream, j);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lact_apply_kernel, dim3((unsigned)((size_t)j.BH * ((j.T + kTok - 1) / kTok))),
                       dim3(kThreads), 0, stream, j);
    return hipGetLastError();
}

}  // namespace gds
