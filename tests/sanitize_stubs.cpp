// Device launchers for the sanitizer build of the host library (tests/test_sanitizers.py):
// the host code is built and linked without the HIP kernels, so these stand in for the
// launch wrappers of the .hip files.  The driver never reaches them (its pools have no
// device storage); if it did, the call fails as on a machine without a GPU.
#include "forkkv_internal.h"

namespace forkkv {

hipError_t launch_decode_generic(const DecodeParams&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_mfma(const DecodeParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_combine(const DecodeParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_write(const PrefillParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_generic(const PrefillParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_mfma(const PrefillParams&, const int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_cow_copy(void*, int, int, int, int32_t, int32_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
void* noalloc_scratch(hipError_t* err) {
  *err = hipErrorNoDevice;
  return nullptr;
}

}  // namespace forkkv
