// blelloch.hip -- long-sequence path (placeholder until the kernels land).
#include "blelloch.hpp"
#include "kernels.hpp"

namespace gds {

int sequential_workgroups_per_head(bool mfma, int dv) { return mfma ? 2 : dv / 16; }
bool blelloch_supported(int, int, int, int, int) { return false; }
int blelloch_default_leaf_chunks(int64_t, int64_t, int) { return 64; }
size_t blelloch_workspace_bytes(int64_t, int64_t, int, int, int) { return 0; }
hipError_t launch_blelloch(int, int, int, int, int, int, int, const void*, const void*,
                           const void*, const float*, const float*, const float*, void*, float*,
                           void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gds
