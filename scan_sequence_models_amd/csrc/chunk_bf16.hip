// chunk_bf16.hip -- bfloat16 MFMA chunk kernel (placeholder).
#include "kernels.hpp"

namespace gds {

bool chunk_mfma_supported(int, int, int, int) { return false; }
hipError_t launch_chunk_mfma(int, int, int, int, int, int, const void*, const void*, const void*,
                             const float*, const float*, const float*, void*, float*,
                             hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gds
