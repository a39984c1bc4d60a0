// The within-chunk inclusive sum of dt * A for one head, computed by one
// wavefront (the blocked algorithm's per-chunk decay; "Mamba-2 vs
// Transformers: SSMs, structured state space duality", section "Mamba-2 and
// the SSD paper: what changed in practice"). Shared by the stand-alone
// cumsum kernel and the chunk-state kernel that fuses it, so both produce the
// same bits.
#pragma once

#include "ssd_internal.h"

namespace ssd {

// dt as the entry points use it: optional per-head bias, softplus
// log(1 + e^z) (z itself above 20, where the two agree in fp32), then an
// optional clamp. Applied to positions inside the sequence only.
__device__ __forceinline__ float dt_pre(float v, int h, const DtOpts& o) {
  if (o.bias != nullptr) v += o.bias[h];
  if (o.softplus) v = v > 20.f ? v : log1pf(expf(v));
  if (o.clamp) v = fminf(fmaxf(v, o.lo), o.hi);
  return v;
}

// Lane `lane` owns the QPL = Q/64 consecutive positions lane*QPL .. +QPL-1 of
// the chunk; d[] holds their dt (0 past the sequence end). On return s[k] is
// the inclusive sum of dt*a over positions 0 .. lane*QPL + k.
template <int QPL>
__device__ __forceinline__ void wave_chunk_cumsum(const float (&d)[QPL], float a, float (&s)[QPL], int lane) {
  float run = 0.f;
#pragma unroll
  for (int k = 0; k < QPL; ++k) {
    run += d[k] * a;
    s[k] = run;
  }
  // inclusive wavefront scan of the lane totals
  float incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  const float excl = incl - run;
#pragma unroll
  for (int k = 0; k < QPL; ++k) s[k] += excl;
}

}  // namespace ssd
