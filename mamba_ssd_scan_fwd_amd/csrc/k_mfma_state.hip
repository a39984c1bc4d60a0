// Step 2 on bf16 matrix cores (placeholder until the MFMA kernel lands).
#include "ssd_internal.h"

namespace ssd {
bool mfma_chunk_state_supported(const Plan&) { return false; }
hipError_t launch_chunk_state_mfma(const Plan&, const void*, const void*, const float*,
                                   const float*, void*, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace ssd
