// Host-only stand-ins for the kernel launchers of libgmlp, for the sanitizer build of the C ABI's
// host code (api.cpp) that the CPU test test_host_sanitizers.py makes: every launcher returns
// success without touching a device, so the validation, sizing and planning code runs under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.  Test code only:
// the library that the package loads is built from the real kernels.
#include "kernels.h"

namespace gmlp {

hipError_t launch_scan(const int32_t*, int, int64_t, SplitTables, hipStream_t) { return hipSuccess; }
hipError_t launch_fill_u32(uint32_t*, uint32_t, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_mxfp8_quant(const uint16_t*, int64_t, int64_t, SplitTables, int, bool, bool, MxOut, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_dact_quant(const DactArgs&, SplitTables, int, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_act_quant(const uint16_t*, const float*, Act, int64_t, SplitTables, int, int64_t, MxOut,
                            hipStream_t) {
  return hipSuccess;
}
hipError_t launch_hadamard_amax(const uint16_t*, int64_t, int64_t, SplitTables, int, uint32_t, float*, float*,
                                hipStream_t, ActSrc) {
  return hipSuccess;
}
hipError_t launch_amax_finalize(SplitTables, int, float*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_nvfp4_quant(const uint16_t*, int64_t, int64_t, SplitTables, int, uint32_t, bool, bool, bool,
                              const float*, const float*, NvOut, hipStream_t, ActSrc) {
  return hipSuccess;
}
hipError_t launch_weight_amax(const uint16_t*, const void* const*, int, int64_t, int64_t, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gather_weights(const void* const*, int, int64_t, int64_t, uint16_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_nv_expand(const uint8_t*, const uint8_t*, uint8_t*, int64_t, int64_t, int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_nv_expand_groups(const uint8_t*, const uint8_t*, uint8_t*, int64_t, int64_t, const int32_t*, int,
                                   hipStream_t) {
  return hipSuccess;
}
hipError_t launch_dact_bf16(const uint16_t*, const uint16_t*, const float*, Act, int64_t, int64_t, uint16_t*,
                            uint16_t*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gemm(const GemmArgs&, hipStream_t) { return hipSuccess; }
int gemm_fprop_ntiles_n(const GemmArgs& g) { return (int)((g.N + 255) / 256); }
hipError_t launch_dprob_reduce(const float*, int, int64_t, float*, hipStream_t) { return hipSuccess; }

}  // namespace gmlp
