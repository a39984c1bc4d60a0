// The short causal convolution's activation, shared by the stand-alone
// convolution kernel and the chunk-state kernel that applies the convolution
// as it loads its tiles, so both produce the same bits.
#pragma once

#include "ssd_internal.h"

namespace ssd {

// z * sigmoid(z), with the hardware reciprocal (about 1 ulp) instead of an
// IEEE division
__device__ __forceinline__ float conv_silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

}  // namespace ssd
