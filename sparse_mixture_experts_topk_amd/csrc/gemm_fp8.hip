// fp8 (e4m3) grouped expert GEMMs -- not yet implemented; the C ABI reports
// MOE_ERR_UNSUPPORTED for fp8 weights before reaching these launchers.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

hipError_t launch_gate_up_fp8(const moe_shape_t&, const uint8_t*, const uint8_t*, const int32_t*,
                              const uint8_t*, const uint8_t*, const float*, const float*, uint8_t*,
                              uint8_t*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_down_fp8(const moe_shape_t&, const uint8_t*, const uint8_t*, const int32_t*,
                           const uint8_t*, const float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
