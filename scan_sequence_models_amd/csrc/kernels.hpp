// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
//
// Every launcher assumes the C-ABI layer has already validated its arguments
// (sizes supported, pointers non-null and aligned) and only enqueues work on
// `stream`.  They return hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gds {

// decode.hip -------------------------------------------------------------
bool decode_supported(int dk);
// mode: 0 gated delta rule, 1 gated linear attention, 2 / 3 the same with
// diagonal gates (alpha [N, dk]).  beta_w: write strengths (the gated delta
// rule's f_t = beta_w v k^T); equal to beta except for split erase/write
// strengths.  Ignored in modes 1 and 3.
hipError_t launch_decode(int mode, int dtype, int N, int dk, int dv, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const float* beta_w, float* S, void* o, hipStream_t stream);

// chunk_f32.hip -- plain float32 chunkwise kernel (any supported size) -------
bool chunk_f32_supported(int mode, int dk, int dv, int chunk);
hipError_t launch_chunk_f32(int mode, int dtype, int BH, int T, int dk, int dv, int chunk,
                            const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* beta_w, const float* S0, void* o,
                            float* ST, hipStream_t stream);

// chunk_diag.hip -- float32 chunkwise kernel with diagonal (per-key-channel) gates
// (mode 0: gated delta rule, 1: gated linear attention; alpha is [BH, T, dk])
bool chunk_diag_supported(int dk, int dv);
hipError_t launch_chunk_diag(int mode, int dtype, int BH, int T, int dk, int dv, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta,
                             const float* S0, void* o, float* ST, hipStream_t stream);

// chunk_bf16.hip -- bfloat16 MFMA chunkwise kernel ---------------------------
// (dk = dv = 128, chunk 64; q, k, v, o bfloat16; states float32)
// kPrism: the sequential pass over PRISM's element stream, read in place (see
// ChunkJob::prism_L)
enum ChunkRole { kSequential = 0, kLeafAggregate = 1, kLeafOutput = 2, kPrism = 3 };

struct ChunkJob {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const float* beta;   // erase strengths (E_t)
    const float* beta_w; // write strengths (f_t); == beta unless split
    uint16_t* o;         // outputs, or null (not written)
    const float* S_in;   // role-dependent, see chunk_bf16.hip
    float* S_out;        // role-dependent, see chunk_bf16.hip
    int heads, T, nchunks;
    int leaves;          // leaves per head
    int leaf_chunks;     // chunks per leaf (the last real leaf may hold fewer)
    int last_leaf;       // kLeafOutput: the leaf whose final state is S_T
    // kPrism: T counts elements, T = prism_T (L + 1).  Element t (L + 1) + l is
    // token t's gated-delta element (l = 0: k, v, alpha, erase and write beta of
    // the token) or its l-th correction (k, v from the factor rows kf, vf
    // [head][prism_T][L][d], alpha 1, erase 0, write beta_l[head][t][l-1]); q_t
    // sits on element l = L, whose output is o_t (o is [head][prism_T][dv]).
    // floor(e / (L + 1)) = mulhi(e, prism_magic) for every element e.
    int prism_L, prism_T;
    unsigned prism_magic;
    const uint16_t* kf;
    const uint16_t* vf;
    const float* beta_l;
};

bool chunk_mfma_supported(int mode, int dk, int dv, int chunk);
hipError_t launch_chunk_job(int mode, int role, const ChunkJob& job, hipStream_t stream);
hipError_t launch_chunk_mfma(int mode, int BH, int T, int dk, int dv, int chunk,
                             const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* beta_w, const float* S0, void* o,
                             float* ST, hipStream_t stream);
// PRISM's element stream scanned in place (bf16, d = 128, 1 <= L <= 8); false if
// T (L + 1) is too long for the element index arithmetic
bool chunk_prism_supported(int T, int L);
hipError_t launch_chunk_prism(int BH, int T, int L, const void* q, const void* k, const void* v,
                              const void* kf, const void* vf, const float* alpha, const float* beta,
                              const float* beta_l, const float* S0, void* o, float* ST,
                              hipStream_t stream);

// scan_bwd.hip -- gradient of the scan through the chunkwise form ------------
struct BwdJob {
    const void *q, *k, *v, *dO;             // element type of dtype; dO may be null (zero)
    const float *alpha, *beta, *S0, *dST;   // beta null for linear attention; S0, dST may be null
    const float* beta_w;                    // write strengths; == beta unless split
    float *dq, *dk_out, *dv_out, *dalpha, *dbeta, *dS0;  // dbeta null for linear attention
    float* dbeta_w;                         // split strengths: gradient of the write plane; else null
    float* ckpt;                            // workspace: states entering each chunk, then partials
    float* part;                            // set by launch_scan_bwd
    int BH, T, dk, dv, nchunks;
};
bool scan_bwd_supported(int dk, int dv);
size_t scan_bwd_workspace_floats(int BH, int T, int dk, int dv);
hipError_t launch_scan_bwd(int mode, int dtype, BwdJob job, hipStream_t stream);

// prism.hip -- PRISM write factors expanded into a split-strength scan stream ---
struct PrismJob {
    const void *q, *k, *v, *x;           // [BH, T, dk] / [BH, T, dv], element type of dtype
    const float *alpha, *beta, *beta_l;  // [BH, T], [BH, T], [BH, T, L]
    const float* conv;                   // [H, W, dv]
    const void *Wk, *Wp;                 // [H, L, dk, dv], [H, L, dv, dv]
    void *q2, *k2, *v2;                  // [BH, T (L+1), d]
    float *alpha2, *beta2;               // [BH, T (L+1)], [2, BH, T (L+1)]
    // compact factor rows instead of the stream (launch_prism_factors):
    void *kf, *vf;                       // [BH, T, L, d]
    int BH, H, T, dk, dv, L, W;
};
bool prism_supported(int dtype, int dk, int dv);
hipError_t launch_prism_expand(int dtype, const PrismJob& job, hipStream_t stream);
// the factor rows k^(l), delta^(l) only, into job.kf, job.vf (bf16, d = 128, L >= 1)
hipError_t launch_prism_factors(const PrismJob& job, hipStream_t stream);

// lact.hip -- large-chunk fast-weight update (linear fast weights) -----------
struct LactJob {
    const void *q, *k, *v;  // [BH, T, dk] / [BH, T, dv]
    const float* eta;       // [BH, T] learning rates
    const float* W0;        // [BH, dv, dk] or null (zero)
    void* o;                // [BH, T, dv]
    float* WT;              // [BH, dv, dk] or null
    float* ws_stats;        // MFMA path: per (head, chunk, split) partial G, F
    uint16_t* ws_wuse;      // MFMA path: per (head, chunk) applied weight, bf16
    int BH, T, dk, dv, chunk, order, nsplit, split_tokens;
};
bool lact_mfma_supported(int dtype, int dk, int dv, int chunk);
bool lact_plain_supported(int dk, int dv);
size_t lact_workspace_bytes(int64_t heads, int T, int chunk);
hipError_t launch_lact(int dtype, LactJob job, void* workspace, hipStream_t stream);

// scratch.hip -- device address of the current device's fixed scratch array
// (SCAN_NOALLOC_MAX_WORKSPACE bytes, 256-byte aligned), looked up once per
// device and cached.  Allocates nothing.
hipError_t noalloc_scratch(void** ptr);

}  // namespace gds
