// blelloch.hip -- long-sequence path: leaf aggregates, a fixed Blelloch tree
// over them, and an output pass that starts every leaf from its prefix state.
//
// "Sequential Parallel Duality in Prefix Scannable Models" (papernotes.org
// notes): training encodes every chunk, runs a static Blelloch scan -- an
// up-sweep that pairs adjacent nodes level by level and a down-sweep that hands
// each chunk its exclusive prefix -- and then reads each chunk out from that
// prefix (overall framework; the worked example fixes the bracketing: (x0,x1)
// and (x2,x3) first, then x_{0:3}).  The monoid is the affine one of key
// design 2; in the right-action form used here an element (E, f) maps a state
// S to S E + f and the combine "a then b" is (E_a E_b, f_a E_b + f_b).
//
// Steps on one stream (heads are independent; a leaf is G consecutive chunks,
// the leaf count m is padded to a power of two with identity leaves):
//  1. leaf pass (chunk kernel, kLeafAggregate): every leaf's (E, f), with f
//     (dv x dk) and E (dk x dk) stored as one 256 x 128 fp32 block [f; E];
//  2. up-sweep, levels 1 .. log2(m)-1: agg_l[k] = agg_{l-1}[2k] then
//     agg_{l-1}[2k+1]  (one 256x128x128 fp32 product per node; the root
//     aggregate feeds no output and is not formed);
//  3. down-sweep on states, top to bottom: the state entering node k of level l
//     is handed unchanged to its left child and as st E_left + f_left to its
//     right child (a 128x128x128 fp32 product); the top state is S0;
//  4. output pass (chunk kernel, kLeafOutput): every leaf from its prefix
//     state, writing o; the last real leaf writes S_T.
// Products of steps 2-3 run on the fp32 MFMA (v_mfma_f32_16x16x4_f32); with
// gated linear attention every E is gamma I and they are scalings.
#include "blelloch.hpp"

#include "common.hpp"
#include "kernels.hpp"

namespace gds {
namespace {

constexpr int D = 128;                    // dk = dv
constexpr size_t kAgg = (size_t)2 * D * D;  // floats per aggregate [f; E]
constexpr size_t kSt = (size_t)D * D;       // floats per state
constexpr int kChunk = 64;

struct Affine {
    // C = A B + F for `rows` rows (128 or 256) and 128 columns, per (head, item);
    // B is 128 x 128; F is added to rows < f_rows only; A == null means zero.
    // D, if set, receives a copy of A (zeros if A is null).
    const float* A; long long a_head, a_item;
    const float* B; long long b_head, b_item;
    const float* F; long long f_head, f_item; int f_rows;
    float* C; long long c_head, c_item;
    float* Dst; long long d_head, d_item;
    int rows, items;
};

constexpr int LDA = D + 4;  // LDS row stride (floats)

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One workgroup: a 64 x 64 block of C.  Wave w owns rows 16w..16w+15 of the
// block and its four 16-column tiles.
__global__ __launch_bounds__(256) void affine_kernel(const Affine p) {
    __shared__ float As[64 * LDA];
    __shared__ float Bt[64 * LDA];  // B block transposed: [column][k]
    const int nrb = p.rows / 64;
    int x = blockIdx.x;
    const int cb = x & 1;
    x >>= 1;
    const int rb = x % nrb;
    x /= nrb;
    const int item = x % p.items;
    const int head = x / p.items;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;

    const float* A = p.A ? p.A + head * p.a_head + item * p.a_item + (size_t)rb * 64 * D : nullptr;
    const float* B = p.B + head * p.b_head + item * p.b_item + cb * 64;
    float* Dst = p.Dst ? p.Dst + head * p.d_head + item * p.d_item + (size_t)rb * 64 * D : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int e = tid + 256 * m;          // 2048 float4 of the 64 x 128 A block
        const int r = e >> 5, c4 = (e & 31) * 4;
        const float4 a = A ? *reinterpret_cast<const float4*>(A + (size_t)r * D + c4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(&As[r * LDA + c4]) = a;
        if (Dst && cb == 0) *reinterpret_cast<float4*>(Dst + (size_t)r * D + c4) = a;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int e = tid + 256 * m;          // 2048 float4 of the 128 x 64 B block
        const int kr = e >> 4, c4 = (e & 15) * 4;
        const float4 b = *reinterpret_cast<const float4*>(B + (size_t)kr * D + c4);
        Bt[(c4 + 0) * LDA + kr] = b.x;
        Bt[(c4 + 1) * LDA + kr] = b.y;
        Bt[(c4 + 2) * LDA + kr] = b.z;
        Bt[(c4 + 3) * LDA + kr] = b.w;
    }
    __syncthreads();

    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    // lane group g supplies k = 16s + 4g + v at sub-step v of step s (same for A and B)
#pragma unroll 2
    for (int s = 0; s < D / 16; ++s) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&As[(16 * w + n16) * LDA + 16 * s + 4 * g4]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(&Bt[(16 * ct + n16) * LDA + 16 * s + 4 * g4]);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[ct] = mfma4(a[v], b[v], acc[ct]);
        }
    }
    float* C = p.C + head * p.c_head + item * p.c_item;
    const float* F = p.F ? p.F + head * p.f_head + item * p.f_item : nullptr;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rb * 64 + 16 * w + 4 * g4 + r;
            const int col = cb * 64 + 16 * ct + n16;
            float val = acc[ct][r];
            if (F && row < p.f_rows) val += F[(size_t)row * D + col];
            C[(size_t)row * D + col] = val;
        }
    }
}

// The same C = A B + F when B is gamma I (gated linear attention: every E is a
// multiple of the identity), so the product is a scaling by B's first entry.
// One workgroup: 64 rows of C.
__global__ __launch_bounds__(256) void affine_scaled_kernel(const Affine p) {
    const int nrb = p.rows / 64;
    int x = blockIdx.x;
    const int rb = x % nrb;
    x /= nrb;
    const int item = x % p.items;
    const int head = x / p.items;
    const float* A = p.A ? p.A + head * p.a_head + item * p.a_item + (size_t)rb * 64 * D : nullptr;
    const float gam = p.B[head * p.b_head + item * p.b_item];
    const float* F = p.F ? p.F + head * p.f_head + item * p.f_item : nullptr;
    float* C = p.C + head * p.c_head + item * p.c_item + (size_t)rb * 64 * D;
    float* Dst = p.Dst ? p.Dst + head * p.d_head + item * p.d_item + (size_t)rb * 64 * D : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int e = threadIdx.x + 256 * m;  // 2048 float4 of the 64 x 128 block
        const int r = e >> 5, c4 = (e & 31) * 4, row = rb * 64 + r;
        const float4 a = A ? *reinterpret_cast<const float4*>(A + (size_t)r * D + c4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        if (Dst) *reinterpret_cast<float4*>(Dst + (size_t)r * D + c4) = a;
        float4 c = make_float4(gam * a.x, gam * a.y, gam * a.z, gam * a.w);
        if (F && row < p.f_rows) {
            const float4 f = *reinterpret_cast<const float4*>(F + (size_t)row * D + c4);
            c.x += f.x; c.y += f.y; c.z += f.z; c.w += f.w;
        }
        *reinterpret_cast<float4*>(C + (size_t)r * D + c4) = c;
    }
}

// Gated linear attention (every E is gamma I).  Sum of ln alpha over leaf i
// of head `head` (tokens [i G C, (i+1) G C) within T), by the threads of one
// workgroup; groups of 256/m lanes per leaf when m <= 64.
__device__ __forceinline__ void leaf_log_decays(const float* alpha, int head, int T, int leaf_tokens, int m,
                                                float* out) {
    __shared__ float part[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (m <= 4) {  // whole waves per leaf
        const int per = 4 / m, li = w / per, sub = w % per;
        const int t0 = li * leaf_tokens, t1 = min(t0 + leaf_tokens, T);
        float s = 0.f;
        for (int t = t0 + sub * 64 + lane; t < t1; t += per * 64) s += __logf(alpha[(size_t)head * T + t]);
        s = group_sum<64>(s);
        if (lane == 0) part[w] = s;
        __syncthreads();
        if (tid < m) {
            float g = 0.f;
            for (int j = 0; j < per; ++j) g += part[tid * per + j];
            out[tid] = g;
        }
    } else {  // m in 8 .. 64: a lane group of G = 256 / m per leaf
        const int G = 256 / m, li = tid / G, sub = tid % G;
        const int t0 = li * leaf_tokens, t1 = min(t0 + leaf_tokens, T);
        float s = 0.f;
        for (int t = t0 + sub; t < t1; t += G) s += __logf(alpha[(size_t)head * T + t]);
        s = G == 32 ? group_sum<32>(s) : G == 16 ? group_sum<16>(s) : G == 8 ? group_sum<8>(s) : group_sum<4>(s);
        if (sub == 0) out[li] = s;
    }
    __syncthreads();
}

// With at most 64 leaves: the state entering each leaf as a left fold over the
// leaves before it, element by element (S_0 = S0, S_{i+1} = gamma_i S_i + f_i);
// the bracketing only changes rounding.  Workgroup (head, block of 1024 state
// elements); the leaves' E rows are not needed.
__global__ __launch_bounds__(256) void gla_prefix_kernel(const float* S0, const float* alpha, const float* agg,
                                                         float* st, int T, int m, int leaf_tokens) {
    __shared__ float lg[64];
    const int head = blockIdx.x / 16, e4 = (blockIdx.x % 16) * 1024 + 4 * threadIdx.x;
    leaf_log_decays(alpha, head, T, leaf_tokens, m, lg);
    float4 cur = S0 ? *reinterpret_cast<const float4*>(S0 + (size_t)head * kSt + e4) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < m; ++i) {
        const size_t leaf = (size_t)head * m + i;
        *reinterpret_cast<float4*>(st + leaf * kSt + e4) = cur;
        const float g = __expf(lg[i]);
        const float4 f = *reinterpret_cast<const float4*>(agg + leaf * kAgg + e4);
        cur = make_float4(g * cur.x + f.x, g * cur.y + f.y, g * cur.z + f.z, g * cur.w + f.w);
    }
}

// With more leaves: E = gamma I written into every leaf aggregate for the
// (scaled) sweeps.  One workgroup per (head, leaf).
__global__ __launch_bounds__(256) void gla_leaf_decay_kernel(const float* alpha, float* agg, int T, int m,
                                                             int leaf_tokens) {
    __shared__ float part[4];
    const int u = blockIdx.x, tid = threadIdx.x;
    const int head = u / m, leaf = u - head * m;
    const int t0 = leaf * leaf_tokens, t1 = min(t0 + leaf_tokens, T);
    float s = 0.f;
    for (int t = t0 + tid; t < t1; t += 256) s += __logf(alpha[(size_t)head * T + t]);
    s = group_sum<64>(s);
    if ((tid & 63) == 0) part[tid >> 6] = s;
    __syncthreads();
    const float gam = __expf(part[0] + part[1] + part[2] + part[3]);
    float* E = agg + (size_t)u * kAgg + kSt;
    for (int x = 4 * tid; x < D * D; x += 4 * 256) {
        const int r = x / D, c = x - r * D;
        *reinterpret_cast<float4*>(E + x) =
            make_float4(c == r ? gam : 0.f, c + 1 == r ? gam : 0.f, c + 2 == r ? gam : 0.f, c + 3 == r ? gam : 0.f);
    }
}

hipError_t launch_affine(const Affine& p, int heads, bool scaled, hipStream_t s) {
    const unsigned rblocks = (unsigned)(heads * p.items * (p.rows / 64));
    if (scaled)
        hipLaunchKernelGGL(affine_scaled_kernel, dim3(rblocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(affine_kernel, dim3(rblocks * 2), dim3(256), 0, s, p);
    return hipGetLastError();
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t next_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p *= 2;
    return p;
}

struct Layout {
    int64_t m;            // leaves per head (power of two)
    int levels;           // log2(m)
    size_t agg_off[40];   // float offsets of aggregate levels 0 .. levels-1
    size_t st_off[40];    // float offsets of state levels 0 .. levels-1
    size_t floats;
};

Layout layout(int64_t heads, int64_t nchunks, int leaf_chunks) {
    Layout L{};
    L.m = next_pow2(ceil_div(nchunks, leaf_chunks));
    while ((int64_t(1) << L.levels) < L.m) ++L.levels;
    size_t off = 0;
    for (int l = 0; l < L.levels; ++l) {
        L.agg_off[l] = off;
        off += (size_t)heads * (size_t)(L.m >> l) * kAgg;
    }
    for (int l = 0; l < L.levels; ++l) {
        L.st_off[l] = off;
        off += (size_t)heads * (size_t)(L.m >> l) * kSt;
    }
    L.floats = off;
    return L;
}

}  // namespace

int sequential_workgroups_per_head(bool mfma, int dv) { return mfma ? 2 : dv / 16; }

bool blelloch_supported(int mode, int dtype, int dk, int dv, int chunk) {
    return dtype == 1 && chunk_mfma_supported(mode, dk, dv, chunk) && dk == D && dv == D;
}

int blelloch_default_leaf_chunks(int64_t nchunks, int64_t heads, int cus) {
    // enough leaves that the output pass (2 workgroups per leaf) fills every CU
    // about once (the leaf pass, 4 workgroups per leaf, twice), and at least 16
    // chunks per leaf; measured best for 16 heads x 4096 chunks and 32 heads x
    // 64 chunks on 256 CUs (fewer, longer leaves also shorten the tree)
    int64_t leaves = next_pow2(ceil_div((int64_t)cus, 2 * heads));
    while (leaves > 1 && nchunks / leaves < 16) leaves >>= 1;
    int64_t g = next_pow2(ceil_div(nchunks, leaves));
    if (g < 1) g = 1;
    if (g > (1 << 20)) g = 1 << 20;
    return (int)g;
}

size_t blelloch_workspace_bytes(int64_t heads, int64_t nchunks, int leaf_chunks, int dk, int dv) {
    (void)dk; (void)dv;
    const Layout L = layout(heads, nchunks, leaf_chunks);
    return L.floats * sizeof(float);
}

hipError_t launch_blelloch(int mode, int BH, int T, int dk, int dv, int chunk, int leaf_chunks,
                           const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* beta_w, const float* S0, void* o,
                           float* ST, void* workspace, hipStream_t stream) {
    const int nchunks = (T + kChunk - 1) / kChunk;
    const Layout L = layout(BH, nchunks, leaf_chunks);
    if (L.m == 1)  // one leaf: the tree is empty
        return launch_chunk_mfma(mode, BH, T, dk, dv, chunk, q, k, v, alpha, beta, beta_w, S0, o, ST,
                                 stream);
    float* ws = static_cast<float*>(workspace);

    ChunkJob job{};
    job.q = static_cast<const uint16_t*>(q);
    job.k = static_cast<const uint16_t*>(k);
    job.v = static_cast<const uint16_t*>(v);
    job.alpha = alpha;
    job.beta = beta;
    job.beta_w = beta_w;
    job.heads = BH;
    job.T = T;
    job.nchunks = nchunks;
    job.leaves = (int)L.m;
    job.leaf_chunks = leaf_chunks;
    job.last_leaf = (nchunks - 1) / leaf_chunks;

    // 1. leaf aggregates
    job.o = nullptr;
    job.S_in = nullptr;
    job.S_out = ws + L.agg_off[0];
    hipError_t e = launch_chunk_job(mode, kLeafAggregate, job, stream);
    if (e != hipSuccess) return e;
    const int leaf_tokens = leaf_chunks * kChunk;
    if (mode == 1 && L.m <= 64) {
        // gated linear attention: a left fold per state element replaces the sweeps
        hipLaunchKernelGGL(gla_prefix_kernel, dim3((unsigned)(BH * 16)), dim3(256), 0, stream, S0, alpha,
                           ws + L.agg_off[0], ws + L.st_off[0], T, (int)L.m, leaf_tokens);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        if (mode == 1) {
            hipLaunchKernelGGL(gla_leaf_decay_kernel, dim3((unsigned)(BH * L.m)), dim3(256), 0, stream, alpha,
                               ws + L.agg_off[0], T, (int)L.m, leaf_tokens);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }

    // 2. up-sweep
    for (int l = 1; l < L.levels; ++l) {
        const long long nl = L.m >> l, np = L.m >> (l - 1);
        Affine p{};
        p.A = ws + L.agg_off[l - 1];
        p.a_head = np * kAgg; p.a_item = 2 * kAgg;
        p.B = ws + L.agg_off[l - 1] + kAgg + kSt;           // E rows of the right child
        p.b_head = np * kAgg; p.b_item = 2 * kAgg;
        p.F = ws + L.agg_off[l - 1] + kAgg;                 // f rows of the right child
        p.f_head = np * kAgg; p.f_item = 2 * kAgg; p.f_rows = D;
        p.C = ws + L.agg_off[l];
        p.c_head = nl * kAgg; p.c_item = kAgg;
        p.rows = 2 * D;
        p.items = (int)nl;
        if ((e = launch_affine(p, BH, mode == 1, stream)) != hipSuccess) return e;
    }

    // 3. down-sweep on states
    for (int l = L.levels; l >= 1; --l) {
        const long long nl = L.m >> l, nc = L.m >> (l - 1);
        Affine p{};
        if (l == L.levels) {
            p.A = S0;  // may be null: zero initial state
            p.a_head = (long long)kSt; p.a_item = 0;
        } else {
            p.A = ws + L.st_off[l];
            p.a_head = nl * kSt; p.a_item = kSt;
        }
        p.B = ws + L.agg_off[l - 1] + kSt;                  // E rows of the left child
        p.b_head = nc * kAgg; p.b_item = 2 * kAgg;
        p.F = ws + L.agg_off[l - 1];                        // f rows of the left child
        p.f_head = nc * kAgg; p.f_item = 2 * kAgg; p.f_rows = D;
        p.C = ws + L.st_off[l - 1] + kSt;                   // right child
        p.c_head = nc * kSt; p.c_item = 2 * kSt;
        p.Dst = ws + L.st_off[l - 1];                       // left child
        p.d_head = nc * kSt; p.d_item = 2 * kSt;
        p.rows = D;
        p.items = (int)nl;
        if ((e = launch_affine(p, BH, mode == 1, stream)) != hipSuccess) return e;
    }

    }  // sweeps

    // 4. output pass from every leaf's prefix state
    job.o = static_cast<uint16_t*>(o);
    job.S_in = ws + L.st_off[0];
    job.S_out = ST;
    return launch_chunk_job(mode, kLeafOutput, job, stream);
}

}  // namespace gds
