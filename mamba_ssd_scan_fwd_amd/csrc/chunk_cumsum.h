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
// dt_pre_with takes the head's bias already loaded (used only when o.bias
// is set), so that a caller can issue that load early, beside its others.
__device__ __forceinline__ float dt_pre_with(float v, float bias, const DtOpts& o) {
  if (o.bias != nullptr) v += bias;
  if (o.softplus) v = v > 20.f ? v : log1pf(expf(v));
  if (o.clamp) v = fminf(fmaxf(v, o.lo), o.hi);
  return v;
}
__device__ __forceinline__ float dt_pre(float v, int h, const DtOpts& o) {
  return dt_pre_with(v, o.bias != nullptr ? o.bias[h] : 0.f, o);
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

// Packed sequences in fixed chunks: where a sequence starts, the running sum
// takes an extra -kSegJump. The decay between positions on both sides of a
// start, exp(l_i - l_j) with j before it, then has an exponent below -128:
// it is 0 in fp32 (below the smallest subnormal), so no chunk-local product
// mixes two sequences, a chunk's total decay exp(Lam_c) is 0 once a sequence
// starts in it (state passing restarts there), and the entering state's
// factor exp(l_i) is 0 for every position after a start. Within one
// sequence the jumps cancel in every difference.
//
// After k starts the values lie near -128 k, where fp32 resolves steps of
// 2^-16 k and more. A running sum at that size would gather one rounding per
// position; instead each position carries (starts so far, offset A of its
// sequence's first position, sum s of dt*a since then), combined by a
// segmented scan, and is rounded once, l = A + s. Every difference inside a
// sequence is then off by at most one rounding of l.
constexpr float kSegJump = 128.f;

// As wave_chunk_cumsum, with the jumps at the positions where st[k] is set.
// With no start in the chunk the result has wave_chunk_cumsum's bits.
template <int QPL>
__device__ __forceinline__ void wave_chunk_cumsum_jump(const float (&d)[QPL], float a, const bool (&st)[QPL],
                                                       float (&s)[QPL], int lane) {
  // this lane's positions: starts so far, offset (relative to the lane's
  // first position), sum since the last start
  int nk = 0;
  float la = 0.f, run = 0.f;
  int kk[QPL];
  float ka[QPL];
#pragma unroll
  for (int k = 0; k < QPL; ++k) {
    if (st[k]) {
      la = (la + run) - kSegJump;
      run = d[k] * a;
      ++nk;
    } else {
      run += d[k] * a;
    }
    s[k] = run;
    kk[k] = nk;
    ka[k] = la;
  }
  // segmented inclusive scan over the lanes: (k, A, s) of a left part
  // followed by a right part is (kL + kR, kR ? AL + sL + AR : AL, kR ? sR : sL + sR)
  int ik = nk;
  float ia = la, is = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ok = __shfl_up(ik, off, 64);
    const float oa = __shfl_up(ia, off, 64);
    const float os = __shfl_up(is, off, 64);
    if (lane >= off) {
      if (ik > 0) {
        ia = (oa + os) + ia;
      } else {
        ia = oa;
        is += os;
      }
      ik += ok;
    }
  }
  // the lanes before this one
  const int pk = __shfl_up(ik, 1, 64);
  const float pa = __shfl_up(ia, 1, 64), ps = __shfl_up(is, 1, 64);
  int ek;
  float ea, es;
  if (nk == 0) {  // (as wave_chunk_cumsum where no start precedes)
    ek = ik;
    ea = ia;
    es = is - run;
  } else {
    ek = lane > 0 ? pk : 0;
    ea = lane > 0 ? pa : 0.f;
    es = lane > 0 ? ps : 0.f;
  }
#pragma unroll
  for (int k = 0; k < QPL; ++k) {
    if (kk[k] > 0) {
      s[k] = ((ea + es) + ka[k]) + s[k];
    } else {
      s[k] += es;
      if (ek > 0) s[k] = ea + s[k];
    }
  }
}

}  // namespace ssd
