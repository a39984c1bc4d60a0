// Steps 4+5 on bf16 matrix cores (placeholder until the MFMA kernel lands).
#include "ssd_internal.h"

namespace ssd {
bool mfma_chunk_scan_supported(const Plan&) { return false; }
hipError_t launch_chunk_scan_mfma(const Plan&, const void*, const void*, const void*,
                                  const float*, const float*, const float*, const void*, void*,
                                  hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace ssd
