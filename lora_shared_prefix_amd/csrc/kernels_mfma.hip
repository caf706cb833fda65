// MFMA (matrix-core) ResidualAttention kernels for gfx950.
#include <hip/hip_runtime.h>

#include "forkkv_internal.h"

namespace forkkv {

bool mfma_supported(int dtype, int head_dim, int rank, int group) {
  (void)dtype; (void)head_dim; (void)rank; (void)group;
  return false;
}

int mfma_group_agents(int group) { return group > 0 ? 16 / group : 0; }

bool prefill_mfma_enabled() { return false; }

hipError_t launch_decode_mfma(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_prefill_mfma(const PrefillParams&, const int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace forkkv
