// Host-only stand-ins for the kernel launchers of libmxmoe, linked with the
// C-ABI layer (api.cpp) into a sanitizer build that runs without a GPU.
// Every stub returns an error: a validation test that reaches one means
// that the C-ABI layer let invalid arguments through to a launch, and the
// entry point then reports MX_ERR_HIP instead of the expected code.
#include <hip/hip_runtime.h>

#include "../../mxfp8_block_scaled_04_amd/csrc/mx_internal.h"

namespace mx {

hipError_t launch_quantize_rows(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_quantize_cols(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int32_t, uint8_t*,
                                uint8_t*, int64_t, int32_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_quantize_dual(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int32_t, uint8_t*,
                                uint8_t*, uint8_t*, uint8_t*, int64_t, int32_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_grouped_gemm(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*,
                               int32_t, int64_t, int64_t, int64_t, uint16_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_grouped_gemm_swiglu(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                      const int32_t*, int32_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*,
                                      uint16_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_grouped_gemm_dgrad(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                     const int32_t*, int32_t, int64_t, int64_t, int64_t, int64_t, uint16_t*,
                                     hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_grouped_gemm_wgrad(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                     const int32_t*, int32_t, int64_t, int64_t, int64_t, uint16_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_swiglu_backward(const uint16_t*, const uint16_t*, int64_t, int64_t, uint16_t*, uint16_t*,
                                  hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_validate_offsets(const int32_t*, int32_t, int64_t, int32_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_stream21(const void*, void*, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_swiglu_backward_quant(const uint16_t*, const uint16_t*, int64_t, int64_t, const int32_t*, int32_t,
                                        uint8_t*, uint8_t*, uint8_t*, uint8_t*, uint8_t*, uint8_t*, int64_t, int32_t*,
                                        hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_mfma_probe(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const float*, float*,
                             int32_t, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_route_plan(const int32_t*, const float*, int64_t, int32_t, int32_t, int32_t*, int32_t*, int32_t*,
                             float*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_gather_quantize(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, const float*, int64_t,
                                  const int32_t*, int32_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*, int64_t, int32_t*,
                                  hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_combine(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, const float*, int64_t, int32_t,
                          uint16_t*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace mx
