// The library's own split-K workspace for forkkv_residual_attn_decode_noalloc: a file-scope
// device array of FORKKV_NOALLOC_SCRATCH_BYTES, so that callers that cannot allocate (code
// under stream capture, tight serving loops, harnesses that forbid hipMalloc) need not
// bring a workspace.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code the array's name is only a stand-in; the device address of this GPU's
// copy comes from hipGetSymbolAddress, taken once per device (with that device current) on
// the first call there, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "forkkv_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FORKKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace forkkv {

// Device address of the current device's scratch array; nullptr with the HIP error in *err
// when the device cannot be queried or the symbol not resolved.
void* noalloc_scratch(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_ptr[dev];
}

}  // namespace forkkv
