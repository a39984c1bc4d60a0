// One recurrent step for a batch of sequences (decode): the recurrence itself
// at a single token, with the state kept in HBM between calls ("Mamba-2 vs
// Transformers: SSMs, structured state space duality", table "Evaluation
// criteria ...": the recurrent mode keeps an O(1) per-token state; Telegram
// post "Mamba3": decoding is dominated by moving the state, at about 2.5
// operations per byte). Per (b, h, p):
//     h[p][n] <- exp(dt A_h) h[p][n] + dt x[p] B[n]
//     y[p]     = sum_n h[p][n] C[n] + D_h x[p]
//
// Pure streaming: the fp32 state is read once and written once, everything
// else is small. Each thread owns four consecutive n of one state row (one
// 16-byte load and store), TPR = N/4 threads share a row and reduce y with
// cross-lane shuffles; a thread handles RPT rows so that several loads are in
// flight before the first use.
#include "chunk_cumsum.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kRPT = 2;  // state rows per thread

template <typename TIO> struct IO4;
template <> struct IO4<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <> struct IO4<__hip_bfloat16> {
  static __device__ __forceinline__ float4 load(const __hip_bfloat16* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  }
};

template <typename TIO, int N>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    const TIO* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const TIO* __restrict__ Bm, const TIO* __restrict__ Cm, const float* __restrict__ D,
    float* __restrict__ state, TIO* __restrict__ y, int64_t rows, int H, int pshift, int hpg, DtOpts dto) {
  constexpr int TPR = N / 4;                        // threads per state row
  constexpr int RPW = kThreads / TPR;               // rows per workgroup and pass
  const int tid = threadIdx.x;
  const int sub = tid % TPR;                        // which four n
  const int64_t row0 = (int64_t)blockIdx.x * RPW * kRPT + tid / TPR;

  // Every load of the thread's rows is issued first, from valid addresses
  // only (the optional D and dt bias read A's address when absent and are
  // selected away), so that the thread waits once for all of them instead of
  // once per dependent group.
  float4 hs[kRPT], bv[kRPT], cv[kRPT];
  float dtv[kRPT], av[kRPT], xv[kRPT], dv[kRPT], biv[kRPT];
  int64_t rr[kRPT], rc[kRPT];
  const float* dsrc = D != nullptr ? D : A;
  const float* bsrc = dto.bias != nullptr ? dto.bias : A;
  const int G = H / hpg;
#pragma unroll
  for (int k = 0; k < kRPT; ++k) {
    rr[k] = row0 + (int64_t)k * RPW;
    // rows past the end re-read the last row (not stored)
    const int64_t r = rr[k] < rows ? rr[k] : rows - 1;
    rc[k] = r;
    // row r = (b * H + h) * P + p; P is a power of two and b * H < 2^31
    const int bh = (int)(r >> pshift);
    const int b = bh / H, h = bh - b * H;
    const int g = h / hpg;
    hs[k] = *reinterpret_cast<const float4*>(state + r * N + 4 * sub);
    dtv[k] = dt[bh];
    av[k] = A[h];
    xv[k] = to_f32(x[r]);
    bv[k] = IO4<TIO>::load(Bm + ((int64_t)b * G + g) * N + 4 * sub);
    cv[k] = IO4<TIO>::load(Cm + ((int64_t)b * G + g) * N + 4 * sub);
    dv[k] = dsrc[h];
    biv[k] = bsrc[h];
  }
#pragma unroll
  for (int k = 0; k < kRPT; ++k) {
    const float d = dt_pre_with(dtv[k], biv[k], dto);
    const float alpha = __expf(d * av[k]);
    const float xp = xv[k];
    const float u = d * xp;
    float4 hn;
    hn.x = fmaf(alpha, hs[k].x, u * bv[k].x);
    hn.y = fmaf(alpha, hs[k].y, u * bv[k].y);
    hn.z = fmaf(alpha, hs[k].z, u * bv[k].z);
    hn.w = fmaf(alpha, hs[k].w, u * bv[k].w);
    float part = hn.x * cv[k].x + hn.y * cv[k].y + hn.z * cv[k].z + hn.w * cv[k].w;
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, TPR);
    if (rr[k] < rows) {
      *reinterpret_cast<float4*>(state + rc[k] * N + 4 * sub) = hn;
      if (sub == 0) {
        const float dh = D != nullptr ? dv[k] : 0.f;
        y[rc[k]] = from_f32<TIO>(fmaf(dh, xp, part));
      }
    }
  }
}

template <typename TIO>
hipError_t launch_io(const Plan& p, const void* x, const float* dt, const float* A, const void* B,
                     const void* C, const float* D, float* state, void* y, hipStream_t s) {
  const int64_t rows = p.batch * p.H * p.P;
  auto go = [&](auto kern, int tpr) {
    const int64_t per_wg = (int64_t)(kThreads / tpr) * kRPT;
    const int64_t grid = (rows + per_wg - 1) / per_wg;
    kern<<<dim3((unsigned)grid), kThreads, 0, s>>>(
        static_cast<const TIO*>(x), dt, A, static_cast<const TIO*>(B), static_cast<const TIO*>(C), D, state,
        static_cast<TIO*>(y), rows, (int)p.H, __builtin_ctzll((unsigned long long)p.P), (int)(p.H / p.G), p.dto);
    return hipGetLastError();
  };
  switch (p.N) {
    case 16: return go(decode_step_kernel<TIO, 16>, 4);
    case 32: return go(decode_step_kernel<TIO, 32>, 8);
    case 64: return go(decode_step_kernel<TIO, 64>, 16);
    case 128: return go(decode_step_kernel<TIO, 128>, 32);
    case 256: return go(decode_step_kernel<TIO, 256>, 64);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_step(const Plan& p, const void* x, const float* dt, const float* A, const void* B,
                              const void* C, const float* D, float* state, void* y, hipStream_t s) {
  if (p.io == kBF16) return launch_io<__hip_bfloat16>(p, x, dt, A, B, C, D, state, y, s);
  return launch_io<float>(p, x, dt, A, B, C, D, state, y, s);
}

}  // namespace ssd
