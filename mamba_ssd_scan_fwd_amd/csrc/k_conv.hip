// The short causal convolution in front of the SSM, split into x, B and C.
//
// Mamba-1 and Mamba-2 place a short causal convolution on the input before
// the state-space step (Telegram post "Mamba3", paragraph on the removed short
// causal convolution; "Mamba-3 : SSM optimise inference", section
// "Architecture revisitee": the short conv inherited from H3 and Mamba-1).
// The pages give neither its width nor its activation; this kernel takes
// both as parameters: for every channel ch of the packed token vector
// [x (h, p) | B (g, n) | C (g, n)],
//     z[t][ch] = bias[ch] + sum_{k<K} w[ch][k] * in[t - (K-1) + k][ch]
//     out      = silu ? z * sigmoid(z) : z
// with in[t < 0] taken from the carried convolution state (zeros if none),
// and the last K-1 inputs written out as the state for the next call.
//
// Streaming: each thread owns four consecutive channels (one 8- or 16-byte
// access per token) and walks a tile of kTT tokens, kU tokens' loads at a
// time, keeping the K-1 previous inputs in registers, so every input is read
// once per tile plus a K-1 halo.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kTT = 64;  // tokens per tile
constexpr int kU = 8;    // tokens whose loads are issued together

template <typename T> struct V4;
template <> struct V4<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct V4<__hip_bfloat16> {
  static __device__ __forceinline__ float4 load(const __hip_bfloat16* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  }
  static __device__ __forceinline__ void store(__hip_bfloat16* p, float4 v) {
    auto b = [](float f) { return (uint32_t)__bfloat16_as_ushort(__float2bfloat16(f)); };
    *reinterpret_cast<uint2*>(p) = make_uint2(b(v.x) | (b(v.y) << 16), b(v.z) | (b(v.w) << 16));
  }
};

// z * sigmoid(z), with the hardware reciprocal (about 1 ulp) instead of an
// IEEE division
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

template <typename TIO, int K>
__global__ __launch_bounds__(kThreads) void conv1d_split_kernel(
    const TIO* __restrict__ xbc, const float* __restrict__ w, const float* __restrict__ bias, int act,
    const float* __restrict__ st_in, float* __restrict__ st_out,
    TIO* __restrict__ xo, TIO* __restrict__ bo, TIO* __restrict__ co,
    int64_t L, int XC, int BC) {
  const int CH = XC + 2 * BC;  // channels: x, then B, then C
  const int ch = 4 * (blockIdx.x * kThreads + threadIdx.x);
  if (ch >= CH) return;
  const int64_t t0 = (int64_t)blockIdx.y * kTT;
  const int64_t b = blockIdx.z;
  const TIO* in = xbc + b * L * CH + ch;

  // Every load below is issued from a valid address and its value selected
  // afterwards (no load behind a branch: a branch join would wait for it),
  // so the weights, bias, history and first tokens are in flight together.
  float4 wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k)
    wk[k] = make_float4(w[(ch + 0) * K + k], w[(ch + 1) * K + k], w[(ch + 2) * K + k], w[(ch + 3) * K + k]);
  const float* bp = bias != nullptr ? bias : w;  // w: any valid address
  const float4 braw = make_float4(bp[ch], bp[ch + 1], bp[ch + 2], bp[ch + 3]);
  const float4 bv = bias != nullptr ? braw : make_float4(0.f, 0.f, 0.f, 0.f);

  // history: the K-1 inputs before t0 (from the carried state before t = 0)
  float4 hist[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int64_t t = t0 - (K - 1) + k;
    const float4 v = V4<TIO>::load(in + (t >= 0 ? t : 0) * CH);
    int j = (int)(t + (K - 1));  // position inside the carried state (clamped: always a valid address)
    j = j < 0 ? 0 : (j > K - 2 ? K - 2 : j);
    const float* s = st_in != nullptr ? st_in + (b * CH + ch) * (K - 1) + j : w;
    const float4 sv = make_float4(s[0], s[K - 1], s[2 * (K - 1)], s[3 * (K - 1)]);
    hist[k] = t >= 0 ? v : (st_in != nullptr ? sv : make_float4(0.f, 0.f, 0.f, 0.f));
  }

  // output channel block: x, B or C (four channels never straddle them)
  TIO* out;
  int64_t ostride;
  if (ch < XC) {
    out = xo + b * L * XC + ch;
    ostride = XC;
  } else if (ch < XC + BC) {
    out = bo + b * L * BC + (ch - XC);
    ostride = BC;
  } else {
    out = co + b * L * BC + (ch - XC - BC);
    ostride = BC;
  }

  const int64_t tend = t0 + kTT < L ? t0 + kTT : L;
  // kU tokens' loads in flight at once (rows past the end re-read the last),
  // the next kU issued before the current ones are used
  float4 nxt[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t t = t0 + u < tend ? t0 + u : tend - 1;
    nxt[u] = V4<TIO>::load(in + t * CH);
  }
  for (int64_t tb = t0; tb < tend; tb += kU) {
    float4 cur[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) cur[u] = nxt[u];
    // (issued on every pass, past the end too: a load behind a branch would
    // be waited for where the branch joins)
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t t = tb + kU + u < tend ? tb + kU + u : tend - 1;
      nxt[u] = V4<TIO>::load(in + t * CH);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (tb + u < tend) {
        float4 z = bv;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float4 v = k < K - 1 ? hist[k] : cur[u];
          z.x = fmaf(wk[k].x, v.x, z.x);
          z.y = fmaf(wk[k].y, v.y, z.y);
          z.z = fmaf(wk[k].z, v.z, z.z);
          z.w = fmaf(wk[k].w, v.w, z.w);
        }
        if (act) z = make_float4(silu(z.x), silu(z.y), silu(z.z), silu(z.w));
        V4<TIO>::store(out + (tb + u) * ostride, z);
#pragma unroll
        for (int k = 0; k + 1 < K - 1; ++k) hist[k] = hist[k + 1];
        if (K > 1) hist[K > 1 ? K - 2 : 0] = cur[u];
      }
    }
  }

  // the last K-1 inputs, as the state for the next call (the tile that holds
  // the end of the sequence writes it; earlier inputs may come from st_in)
  if (st_out != nullptr && K > 1 && t0 <= L - 1 && L - 1 < t0 + kTT) {
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
      float* s = st_out + (b * CH + ch) * (K - 1) + k;
      s[0] = hist[k].x;
      s[K - 1] = hist[k].y;
      s[2 * (K - 1)] = hist[k].z;
      s[3 * (K - 1)] = hist[k].w;
    }
  }
}

template <typename TIO>
hipError_t launch_io(const Plan& p, int K, const void* xbc, const float* w, const float* bias, int act,
                     const float* st_in, float* st_out, void* x, void* B, void* C, hipStream_t s) {
  const int XC = (int)(p.H * p.P), BC = (int)(p.G * p.N);
  const int CH = XC + 2 * BC;
  dim3 grid((unsigned)((CH / 4 + kThreads - 1) / kThreads), (unsigned)((p.L + kTT - 1) / kTT), (unsigned)p.batch);
  auto go = [&](auto kern) {
    kern<<<grid, kThreads, 0, s>>>(static_cast<const TIO*>(xbc), w, bias, act, st_in, st_out,
                                   static_cast<TIO*>(x), static_cast<TIO*>(B), static_cast<TIO*>(C), p.L, XC, BC);
    return hipGetLastError();
  };
  switch (K) {
    case 1: return go(conv1d_split_kernel<TIO, 1>);
    case 2: return go(conv1d_split_kernel<TIO, 2>);
    case 3: return go(conv1d_split_kernel<TIO, 3>);
    case 4: return go(conv1d_split_kernel<TIO, 4>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv1d_split(const Plan& p, int K, const void* xbc, const float* w, const float* bias, int act,
                               const float* st_in, float* st_out, void* x, void* B, void* C, hipStream_t s) {
  if (p.io == kBF16) return launch_io<__hip_bfloat16>(p, K, xbc, w, bias, act, st_in, st_out, x, B, C, s);
  return launch_io<float>(p, K, xbc, w, bias, act, st_in, st_out, x, B, C, s);
}

}  // namespace ssd
