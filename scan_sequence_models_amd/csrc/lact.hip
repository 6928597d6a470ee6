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
//                      W in float32 registers, W G on split-bf16 MFMA
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
// tiles each).  Tokens come in tiles of 64, double-buffered in LDS (80 KB: two
// workgroups per CU); eta of token t sits in the padding of row t of the k tile.
__global__ __launch_bounds__(kThreads, 2) void lact_stats_kernel(const LactJob j) {
    __shared__ uint16_t Ks[2][kTok * kLdt];
    __shared__ uint16_t Vs[2][kTok * kLdt];
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
        if (tid < kTok) *reinterpret_cast<float*>(&Ks[buf][tid * kLdt + kD]) = er;
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
#pragma unroll
            for (int i = 0; i < 8; ++i)
                e8[i] = *reinterpret_cast<const float*>(&K[(16 * s + 8 * (lane >> 5) + i) * kLdt + kD]);
            bf16x8 b[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) b[J] = tr_operand(K, 16 * s, 32 * J, lane);
            bf16x8 gh, gl, fh, fl;
            // rows 32w.. of eta K (read again: indexing b[] by the wave would
            // compile to a select over every element)
            scale_split(tr_operand(K, 16 * s, 32 * w, lane), e8, gh, gl);
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

// Chunk-by-chunk recursion of one head, W_{b+1} = W_b + F_b - W_b G_b.  W stays
// in float32 registers (wave w: rows 32w .. 32w+31, four 32x32 accumulator
// tiles); W G runs on the bf16 MFMA in split form (W_hi G_hi + W_hi G_lo +
// W_lo G_hi, ~16 significant bits per operand) from LDS copies of W (rows) and
// G^T (rows = G's columns), rewritten every chunk.  Each chunk's applied weight
// leaves as bf16 for the apply kernel.
constexpr int kLdr = kD + 8;  // bf16 row stride of the LDS operand copies
__global__ __launch_bounds__(kThreads, 1) void lact_recur_kernel(const LactJob j) {
    __shared__ uint16_t Wh[kD * kLdr], Wl[kD * kLdr];    // W_b rows, split
    __shared__ uint16_t Gh[kD * kLdr], Gl[kD * kLdr];    // G_b^T rows, split
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int nch = (j.T + j.chunk - 1) / j.chunk;
    const size_t wbase = (size_t)bh * kD * kD;
    // element e of tile J of this lane: row 32w + row(e), column 32J + l32
    auto row = [&](int e) { return 32 * w + 8 * (e >> 2) + 4 * hh + (e & 3); };
    f32x16 W[4];
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 16; ++e) W[J][e] = j.W0 ? j.W0[wbase + (size_t)row(e) * kD + 32 * J + l32] : 0.f;
    auto split_store = [&]() {  // W -> Wh, Wl (and its bf16 rounding to the applied weight)
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint16_t hi = f32_to_bf16(W[J][e]);
                Wh[row(e) * kLdr + 32 * J + l32] = hi;
                Wl[row(e) * kLdr + 32 * J + l32] = f32_to_bf16(W[J][e] - bf16_to_f32(hi));
            }
    };
    auto store_use = [&](int cb) {  // Wh (W rounded to bf16) -> applied weight of chunk cb
        uint16_t* dst = j.ws_wuse + (size_t)(bh * nch + cb) * kD * kD;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = (tid >> 4) + 16 * i;
            *reinterpret_cast<uint4*>(dst + r * kD + 8 * (tid & 15)) =
                *reinterpret_cast<const uint4*>(&Wh[r * kLdr + 8 * (tid & 15)]);
        }
    };
    split_store();
    for (int cb = 0; cb < nch; ++cb) {
        const float* st = j.ws_stats + (size_t)(bh * nch + cb) * j.nsplit * 2 * kD * kD;
        __syncthreads();  // previous chunk's operand reads done; Wh/Wl of W_b complete
        if (j.order == 1) store_use(cb);
        // G_b summed over the splits, transposed into Gh/Gl: thread moves 16
        // float4 of G, four at a time (their loads in flight together)
#pragma unroll 1
        for (int i0 = 0; i0 < 16; i0 += 4) {
            f32x4 gv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i] = *reinterpret_cast<const f32x4*>(st + 4 * (tid + kThreads * (i0 + i)));
            for (int s = 1; s < j.nsplit; ++s) {
                const float* sp = st + (size_t)s * 2 * kD * kD;
#pragma unroll
                for (int i = 0; i < 4; ++i) gv[i] += *reinterpret_cast<const f32x4*>(sp + 4 * (tid + kThreads * (i0 + i)));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = 4 * (tid + kThreads * (i0 + i)), kr = x >> 7, n0 = x & 127;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint16_t hi = f32_to_bf16(gv[i][c]);
                    Gh[(n0 + c) * kLdr + kr] = hi;
                    Gl[(n0 + c) * kLdr + kr] = f32_to_bf16(gv[i][c] - bf16_to_f32(hi));
                }
            }
        }
        __syncthreads();
        // C = W G: A = W rows, B[k][n] = G[k][n] = G^T row n
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            f32x16 c = {};
            const uint16_t* ah = &Wh[(32 * w + l32) * kLdr + 8 * hh];
            const uint16_t* al = &Wl[(32 * w + l32) * kLdr + 8 * hh];
            const uint16_t* bhp = &Gh[(32 * J + l32) * kLdr + 8 * hh];
            const uint16_t* blp = &Gl[(32 * J + l32) * kLdr + 8 * hh];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 a_h = *reinterpret_cast<const bf16x8*>(ah + 16 * kk);
                const bf16x8 a_l = *reinterpret_cast<const bf16x8*>(al + 16 * kk);
                const bf16x8 b_h = *reinterpret_cast<const bf16x8*>(bhp + 16 * kk);
                const bf16x8 b_l = *reinterpret_cast<const bf16x8*>(blp + 16 * kk);
                c = mfma32(a_h, b_h, c);
                c = mfma32(a_h, b_l, c);
                c = mfma32(a_l, b_h, c);
            }
            // W + F - W G in the accumulator layout
            const float* fp = st + kD * kD;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const size_t fi = (size_t)row(e) * kD + 32 * J + l32;
                float fsum = fp[fi];
                for (int s = 1; s < j.nsplit; ++s) fsum += fp[(size_t)s * 2 * kD * kD + fi];
                W[J][e] += fsum - c[e];
            }
        }
        __syncthreads();  // every read of the old Wh/Wl done
        split_store();
        if (j.order == 0) {
            __syncthreads();
            store_use(cb);
        }
    }
    if (j.WT) {
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 16; ++e) j.WT[wbase + (size_t)row(e) * kD + 32 * J + l32] = W[J][e];
    }
}

// O = Q W_use^T for 256 tokens of one head (four tiles of 64 in one chunk):
// wave w computes channels 32w .. 32w+31; its W rows go straight into
// B-operand registers once; q tiles are staged in LDS (the next one in flight
// in registers) and the output is staged in LDS and stored as whole 256-byte
// rows.
constexpr int kLdo = kD + 8;
constexpr int kApplyTiles = 4;
__global__ __launch_bounds__(kThreads, 2) void lact_apply_kernel(const LactJob j) {
    __shared__ uint16_t Qs[kTok * kLdo];
    __shared__ uint16_t Os[kTok * kLdo];
    constexpr int kSpan = kApplyTiles * kTok;
    const int spans = (j.T + kSpan - 1) / kSpan;
    int bh, sp;
    unit_part(blockIdx.x, j.BH, spans, bh, sp);  // a head's spans share its weights via L2
    const int s0 = sp * kSpan;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int nch = (j.T + j.chunk - 1) / j.chunk;
    const uint16_t* q = static_cast<const uint16_t*>(j.q) + (size_t)bh * j.T * kD;
    uint16_t* o = static_cast<uint16_t*>(j.o) + (size_t)bh * j.T * kD;
    uint4 qn[4];
    auto fetch = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + (tid >> 4) + 16 * i;
            qn[i] = t < j.T ? *reinterpret_cast<const uint4*>(q + (size_t)t * kD + 8 * (tid & 15)) : make_uint4(0, 0, 0, 0);
        }
    };
    const int nt = min(kApplyTiles, (j.T - s0 + kTok - 1) / kTok);
    fetch(s0);
    int cb_loaded = -1;
    const int nc = 32 * w + l32;
    bf16x8 b[8];
    for (int it = 0; it < nt; ++it) {
        const int t0 = s0 + it * kTok;
        const int n = min(kTok, j.T - t0);
        __syncthreads();  // previous tile's Qs reads and Os stores done
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&Qs[((tid >> 4) + 16 * i) * kLdo + 8 * (tid & 15)]) = qn[i];
        if (it + 1 < nt) fetch(t0 + kTok);
        const int cb = t0 / j.chunk;  // a 64-token tile lies in one chunk (chunk % 64 == 0)
        if (cb != cb_loaded) {
            const uint16_t* Wu = j.ws_wuse + ((size_t)bh * nch + cb) * kD * kD;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) b[kk] = *reinterpret_cast<const bf16x8*>(Wu + (size_t)nc * kD + 16 * kk + 8 * hh);
            cb_loaded = cb;
        }
        __syncthreads();
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
    hipLaunchKernelGGL(lact_recur_kernel, dim3((unsigned)j.BH), dim3(kThreads), 0, stream, j);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lact_apply_kernel, dim3((unsigned)((size_t)j.BH * ((j.T + kApplyTiles * kTok - 1) / (kApplyTiles * kTok)))),
                       dim3(kThreads), 0, stream, j);
    return hipGetLastError();
}

}  // namespace gds
