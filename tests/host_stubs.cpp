// Stand-ins for the device side of libw4a8 (kernel launches and the static
// scratch lookup) for a host-only build of the C ABI under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Every launch reports hipErrorNoDevice, so
// a call that passes the host-side validation returns W4A8_ERR_DEVICE
// without touching any pointer it was given.
#include <hip/hip_runtime_api.h>

#include "../w4a8_gemm_amd/csrc/kernels.h"

namespace w4a8 {

hipError_t launch_quant_act(const uint16_t*, int, int, int, int8_t*, int, uint16_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_act_static(const uint16_t*, int, int, int, uint16_t, int8_t*, int,
                                   uint16_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemm_skinny(const GemmParams&, int, const SkinnyConfig&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemm_tiled(const GemmParams&, int, const TiledConfig&, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_split_reduce(const GemmParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_w4a16_skinny(const Gemm16Params&, int, const SkinnyConfig&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_w4a16_tiled(const Gemm16Params&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm_fused(const GemmParams&, const uint16_t*, int, int, const SkinnyConfig&,
                             hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_read_probe(const void*, size_t, int, uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t scratch_address(void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}

}  // namespace w4a8
