// Step 3: inter-chunk state passing.
//
// After every chunk's local state S_c is known (computed in parallel), the
// states are recombined in chunk order ("Mamba-2 vs Transformers: SSMs,
// structured state space duality", section "Mamba-2 and the SSD paper: what
// changed in practice"):
//     H_{-1} = h0,   Hin_c = H_{c-1},   H_c = exp(Lam_c) H_{c-1} + S_c,
// where Lam_c is the chunk's total log-decay (last entry of dA_cumsum).
// Hin_c overwrites S_c in place; H_{nc-1} is the final state (fp32).
//
// This is pure streaming: P*N independent lanes per (b, h), sequential over
// chunks, HBM-bound (read S once, write Hin once). Design:
//  * each thread owns VEC consecutive state elements, so every chunk step is
//    one 16-byte load and one 16-byte store per thread (bf16 states) and
//    consecutive threads touch consecutive addresses;
//  * the loads of the next PF chunks are in flight while the current chunk is
//    combined (a register ring, fully unrolled), because the chunk loop is a
//    dependent chain and, with few (b, h) rows, the memory parallelism has to
//    come from inside each thread;
//  * the per-chunk decay exp(Lam_c) is computed once per 64 chunks by the 64
//    lanes of a wavefront (one chunk per lane) and broadcast to the whole
//    wavefront with readlane at each step.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;

template <typename TS> struct Vec8;
template <> struct Vec8<float> {
  float4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const float4*>(p);
    hi = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void to(float* v) const {
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  }
  __device__ __forceinline__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct Vec8<__hip_bfloat16> {
  uint4 raw;
  __device__ __forceinline__ void load(const __hip_bfloat16* p) {
    raw = *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ void to(float* v) const {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(__hip_bfloat16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = __bfloat16_as_ushort(__float2bfloat16(v[2 * k]));
      const uint32_t hi = __bfloat16_as_ushort(__float2bfloat16(v[2 * k + 1]));
      w[k] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// One chain per block row: chain bh = b*H + h walks chunks [0, nc) of its
// sequence; with packed sequences (seqtab != nullptr, batch 1) chain
// bh = s*H + h walks the seqtab[s].y chunk slots from seqtab[s].x of head h,
// so every sequence is a chain of its own. h0 and hT are indexed by the chain.
template <typename TS, int PF>
__global__ __launch_bounds__(kThreads) void state_passing_kernel(
    TS* __restrict__ states, const float* __restrict__ dA_cs,
    const float* h0, float* hT,  // may be the same buffer (in-place update)
    int64_t nc, int Q, int PN, int H, const int2* __restrict__ seqtab) {
  const int64_t bh = blockIdx.x;
  const int e0 = (blockIdx.y * kThreads + threadIdx.x) * kVec;
  const bool active = e0 < PN;
  const int lane = threadIdx.x & 63;

  // this chain's chunks: states / dA_cs rows of (b, h) = row, slots [c_beg, c_beg + cnt)
  int64_t row = bh, c_beg = 0, cnt = nc;
  if (seqtab != nullptr) {
    const int2 st = seqtab[bh / H];
    row = bh % H;
    c_beg = st.x;
    cnt = st.y;
  }

  float h[kVec];
  if (active && h0 != nullptr) {
    Vec8<float> v;
    v.load(h0 + bh * PN + e0);
    v.to(h);
  } else {
#pragma unroll
    for (int k = 0; k < kVec; ++k) h[k] = 0.f;
  }

  TS* s = states + (row * nc + c_beg) * (int64_t)PN + e0;
  const float* lam = dA_cs + (row * nc + c_beg) * Q + (Q - 1);

  Vec8<TS> ring[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k)
    if (active && k < cnt) ring[k].load(s + (int64_t)k * PN);

  float dec = 0.f;
  for (int64_t c0 = 0; c0 < cnt; c0 += PF) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int64_t c = c0 + k;
      if (c < cnt) {
        if ((c & 63) == 0) {  // refresh: lane l holds exp(Lam_{c+l})
          const int64_t cl = c + lane;
          dec = cl < cnt ? __expf(lam[cl * Q]) : 0.f;
        }
        const float d = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(dec), (int)(c & 63)));
        if (active) {
          float sv[kVec];
          ring[k].to(sv);
          if (c + PF < cnt) ring[k].load(s + (c + PF) * PN);
          Vec8<TS>::store(s + c * PN, h);
#pragma unroll
          for (int e = 0; e < kVec; ++e) h[e] = fmaf(d, h[e], sv[e]);
        }
      }
    }
  }
  if (active && hT != nullptr) Vec8<float>::store(hT + bh * PN + e0, h);
}

template <typename TS>
hipError_t launch_typed(const Plan& p, void* states, const float* dA_cs,
                        const float* h0, float* hT, hipStream_t s) {
  const int PN = (int)(p.P * p.N);
  const int64_t chains = p.seqtab != nullptr ? p.nseq * p.H : p.batch * p.H;
  dim3 grid((unsigned)chains, (unsigned)((PN + kThreads * kVec - 1) / (kThreads * kVec)));
  state_passing_kernel<TS, 8><<<grid, kThreads, 0, s>>>(
      static_cast<TS*>(states), dA_cs, h0, hT, p.nc, p.Q, PN, (int)p.H, p.seqtab);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_passing(const Plan& p, void* states, const float* dA_cs,
                                const float* h0, float* hT, hipStream_t s) {
  if (p.io == kBF16) return launch_typed<__hip_bfloat16>(p, states, dA_cs, h0, hT, s);
  return launch_typed<float>(p, states, dA_cs, h0, hT, s);
}

}  // namespace ssd
