// MFMA grouped GEMM for prefill shapes (not built yet: the call reports
// "not supported" so that a forced MFMA path fails loudly).
#include "moe_internal.h"

namespace moe {
bool mfma_available() { return false; }
hipError_t launch_proj_mfma(const ProjArgs&, int, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace moe
