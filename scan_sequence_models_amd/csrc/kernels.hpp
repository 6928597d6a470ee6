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
hipError_t launch_decode(int mode, int dtype, int N, int dk, int dv, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         float* S, void* o, hipStream_t stream);

// chunk_f32.hip -- plain float32 chunkwise kernel (any supported size) -------
bool chunk_f32_supported(int mode, int dk, int dv, int chunk);
hipError_t launch_chunk_f32(int mode, int dtype, int BH, int T, int dk, int dv, int chunk,
                            const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* S0, void* o, float* ST,
                            hipStream_t stream);

// chunk_bf16.hip -- bfloat16 MFMA chunkwise kernel ---------------------------
// (dk = dv = 128, chunk 64; q, k, v, o bfloat16; states float32)
enum ChunkRole { kSequential = 0, kLeafAggregate = 1, kLeafOutput = 2 };

struct ChunkJob {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const float* beta;
    uint16_t* o;         // outputs, or null (not written)
    const float* S_in;   // role-dependent, see chunk_bf16.hip
    float* S_out;        // role-dependent, see chunk_bf16.hip
    int heads, T, nchunks;
    int leaves;          // leaves per head
    int leaf_chunks;     // chunks per leaf (the last real leaf may hold fewer)
    int last_leaf;       // kLeafOutput: the leaf whose final state is S_T
};

bool chunk_mfma_supported(int mode, int dk, int dv, int chunk);
hipError_t launch_chunk_job(int mode, int role, const ChunkJob& job, hipStream_t stream);
hipError_t launch_chunk_mfma(int mode, int BH, int T, int dk, int dv, int chunk,
                             const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, void* o, float* ST,
                             hipStream_t stream);

}  // namespace gds
