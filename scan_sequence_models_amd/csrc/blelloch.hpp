// blelloch.hpp -- host-side interface of the long-sequence (Blelloch) path.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gds {

// Workgroups the sequential path launches per head (value-row slices).
int sequential_workgroups_per_head(bool mfma, int dv);

bool blelloch_supported(int mode, int dtype, int dk, int dv, int chunk);
int blelloch_default_leaf_chunks(int64_t nchunks, int64_t heads, int cus);
size_t blelloch_workspace_bytes(int64_t heads, int64_t nchunks, int leaf_chunks, int dk, int dv);
hipError_t launch_blelloch(int mode, int BH, int T, int dk, int dv, int chunk, int leaf_chunks,
                           const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* beta_w, const float* S0, void* o,
                           float* ST, void* workspace, hipStream_t stream);

}  // namespace gds
