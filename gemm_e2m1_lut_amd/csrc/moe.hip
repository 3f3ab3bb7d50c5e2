// moe.hip -- MXFP4 mixture-of-experts layer (mxfp4_moe_gemm). Not built yet:
// the entry point reports a launch error until the grouped MFMA kernels land.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {

size_t moe_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t) { return 256; }

hipError_t launch_moe(const uint16_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                      const uint8_t*, const int32_t*, const float*, uint16_t*, void*, int64_t,
                      int64_t, int64_t, int64_t, int64_t, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace e2m1
