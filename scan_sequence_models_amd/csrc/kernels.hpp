// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
//
// Every launcher assumes the C-ABI layer has already validated its arguments
// (sizes supported, pointers non-null and aligned) and only enqueues work on
// `stream`.  They return hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

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
bool chunk_mfma_supported(int mode, int dk, int dv, int chunk);
hipError_t launch_chunk_mfma(int mode, int BH, int T, int dk, int dv, int chunk,
                             const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, void* o, float* ST,
                             hipStream_t stream);

}  // namespace gds
