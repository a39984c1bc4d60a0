// Steps 2 and 4+5 with plain fp32 FMA arithmetic (no matrix cores).
//
// These kernels serve the fp32 io dtype, whose accuracy bar (1e-4 relative)
// rules out bf16 matrix-core operands. They follow the same chunked
// decomposition as the matrix-core kernels ("Mamba-2 vs Transformers: SSMs,
// structured state space duality", section "Mamba-2 and the SSD paper: what
// changed in practice"), staging tiles in LDS and accumulating in fp32.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Step 2: states[b,h,c][p][n] = sum_j w_j x_j[p] B_j[n],  w_j = exp(Lam - l_j) dt_j
// One workgroup per (chunk, b*H + h). The P*N outputs are covered in passes
// of kThreads*kAcc; the chunk is walked in tiles of kJT positions.
// ---------------------------------------------------------------------------
constexpr int kJT = 32;
constexpr int kAcc = 8;

template <typename TIO>
__global__ __launch_bounds__(kThreads) void chunk_state_simt_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ Bm,
    const float* __restrict__ dA_cs, const float* __restrict__ dtc,
    TIO* __restrict__ states, int64_t L, int H, int G, int P, int N, int Q, int64_t nc,
    const ChunkInfo* __restrict__ ctab) {
  __shared__ float w[256];
  __shared__ float xs[kJT][128 + 1];
  __shared__ float bs[kJT][256 + 1];
  const int64_t c = blockIdx.x % nc;
  const int64_t bh = blockIdx.x / nc;
  const int64_t b = bh / H;
  const int h = (int)(bh % H);
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  int64_t row0;
  int rows;
  chunk_span(ctab, b, c, L, Q, row0, rows);
  if (rows <= 0) return;  // unused slot of a packed-sequence table (uniform)
  const float* lc = dA_cs + (bh * nc + c) * Q;
  const float* dc = dtc + (bh * nc + c) * Q;
  const float lam = lc[Q - 1];
  for (int j = tid; j < Q; j += kThreads) w[j] = __expf(lam - lc[j]) * dc[j];
  const int PN = P * N;
  TIO* out = states + (bh * nc + c) * (int64_t)PN;

  for (int og = 0; og < PN; og += kThreads * kAcc) {
    float acc[kAcc];
#pragma unroll
    for (int k = 0; k < kAcc; ++k) acc[k] = 0.f;
    for (int j0 = 0; j0 < Q; j0 += kJT) {
      __syncthreads();
      for (int idx = tid; idx < kJT * P; idx += kThreads) {
        const int j = idx / P, p = idx % P;
        const int tl = j0 + j;
        xs[j][p] = tl < rows ? w[j0 + j] * to_f32(x[((row0 + tl) * H + h) * P + p]) : 0.f;
      }
      for (int idx = tid; idx < kJT * N; idx += kThreads) {
        const int j = idx / N, n = idx % N;
        const int tl = j0 + j;
        bs[j][n] = tl < rows ? to_f32(Bm[((row0 + tl) * G + g) * N + n]) : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kAcc; ++k) {
        const int o = og + k * kThreads + tid;
        if (o < PN) {
          const int p = o / N, n = o % N;
          float s = 0.f;
#pragma unroll 8
          for (int j = 0; j < kJT; ++j) s = fmaf(xs[j][p], bs[j][n], s);
          acc[k] += s;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kAcc; ++k) {
      const int o = og + k * kThreads + tid;
      if (o < PN) out[o] = from_f32<TIO>(acc[k]);
    }
  }
}

// ---------------------------------------------------------------------------
// Steps 4+5: for rows i of the chunk,
//   y_i[p] = exp(l_i) sum_n C_i[n] Hin[p][n]
//          + sum_{j<=i} (sum_n C_i[n] B_j[n]) exp(l_i - l_j) dt_j x_j[p]
//          + D_h x_i[p].
// One workgroup per (row block of kIB rows of one chunk, b*H + h).
// ---------------------------------------------------------------------------
constexpr int kIB = 32;
constexpr int kJT2 = 16;
constexpr int kAcc2 = 16;  // kIB * 128 / kThreads

template <typename TIO>
__global__ __launch_bounds__(kThreads) void chunk_scan_simt_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ Bm, const TIO* __restrict__ Cm,
    const float* __restrict__ D, const float* __restrict__ dA_cs,
    const float* __restrict__ dtc, const TIO* __restrict__ states, TIO* __restrict__ y,
    int64_t L, int H, int G, int P, int N, int Q, int64_t nc, const ChunkInfo* __restrict__ ctab) {
  __shared__ float cs[kIB][256 + 1];
  __shared__ float bs[kJT2][256 + 1];
  __shared__ float xs[kJT2][128 + 1];
  __shared__ float gs[kIB][kJT2 + 1];
  __shared__ float li[kIB];
  __shared__ float lj[kJT2], dj[kJT2];
  const int nib = Q / kIB;
  const int64_t blk = blockIdx.x % (nc * nib);
  const int64_t c = blk / nib;
  const int i0 = (int)(blk % nib) * kIB;
  const int64_t bh = blockIdx.x / (nc * nib);
  const int64_t b = bh / H;
  const int h = (int)(bh % H);
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const float* lc = dA_cs + (bh * nc + c) * Q;
  const float* dc = dtc + (bh * nc + c) * Q;
  const TIO* hin = states + (bh * nc + c) * (int64_t)P * N;
  int64_t row0;
  int rows;
  chunk_span(ctab, b, c, L, Q, row0, rows);
  if (i0 >= rows) return;  // whole row block past the end (uniform per block)

  for (int idx = tid; idx < kIB * N; idx += kThreads) {
    const int r = idx / N, n = idx % N;
    const int tl = i0 + r;
    cs[r][n] = tl < rows ? to_f32(Cm[((row0 + tl) * G + g) * N + n]) : 0.f;
  }
  for (int r = tid; r < kIB; r += kThreads) li[r] = lc[i0 + r];
  __syncthreads();

  // outputs o = k*kThreads + tid over the kIB x P block (P <= 128)
  float acc[kAcc2];
#pragma unroll
  for (int k = 0; k < kAcc2; ++k) {
    acc[k] = 0.f;
    const int o = k * kThreads + tid;
    if (o < kIB * P) {
      const int r = o / P, p = o % P;
      float s = 0.f;
      for (int n = 0; n < N; ++n) s = fmaf(cs[r][n], to_f32(hin[(int64_t)p * N + n]), s);
      acc[k] = __expf(li[r]) * s;
    }
  }

  const int jend = i0 + kIB;  // causal: j <= i < i0 + kIB
  for (int j0 = 0; j0 < jend; j0 += kJT2) {
    __syncthreads();
    for (int idx = tid; idx < kJT2 * N; idx += kThreads) {
      const int j = idx / N, n = idx % N;
      const int tl = j0 + j;
      bs[j][n] = tl < rows ? to_f32(Bm[((row0 + tl) * G + g) * N + n]) : 0.f;
    }
    for (int idx = tid; idx < kJT2 * P; idx += kThreads) {
      const int j = idx / P, p = idx % P;
      const int tl = j0 + j;
      xs[j][p] = tl < rows ? to_f32(x[((row0 + tl) * H + h) * P + p]) : 0.f;
    }
    for (int j = tid; j < kJT2; j += kThreads) {
      lj[j] = lc[j0 + j];
      dj[j] = dc[j0 + j];
    }
    __syncthreads();
    for (int idx = tid; idx < kIB * kJT2; idx += kThreads) {
      const int r = idx / kJT2, j = idx % kJT2;
      const int i = i0 + r, jj = j0 + j;
      float v = 0.f;
      if (jj <= i) {
        float s = 0.f;
        for (int n = 0; n < N; ++n) s = fmaf(cs[r][n], bs[j][n], s);
        v = s * __expf(li[r] - lj[j]) * dj[j];
      }
      gs[r][j] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kAcc2; ++k) {
      const int o = k * kThreads + tid;
      if (o < kIB * P) {
        const int r = o / P, p = o % P;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < kJT2; ++j) s = fmaf(gs[r][j], xs[j][p], s);
        acc[k] += s;
      }
    }
  }

  const float dh = D != nullptr ? D[h] : 0.f;
#pragma unroll
  for (int k = 0; k < kAcc2; ++k) {
    const int o = k * kThreads + tid;
    if (o < kIB * P) {
      const int r = o / P, p = o % P;
      const int tl = i0 + r;
      if (tl < rows) {
        const int64_t off = ((row0 + tl) * H + h) * P + p;
        y[off] = from_f32<TIO>(acc[k] + dh * to_f32(x[off]));
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_state_simt(const Plan& p, const void* x, const void* B,
                                   const float* dA_cs, const float* dtc, void* states,
                                   hipStream_t s) {
  dim3 grid((unsigned)(p.nc * p.batch * p.H));
  if (p.io == kBF16) {
    using T = __hip_bfloat16;
    chunk_state_simt_kernel<T><<<grid, kThreads, 0, s>>>(
        static_cast<const T*>(x), static_cast<const T*>(B), dA_cs, dtc, static_cast<T*>(states),
        p.L, (int)p.H, (int)p.G, (int)p.P, (int)p.N, p.Q, p.nc, p.ctab);
  } else {
    chunk_state_simt_kernel<float><<<grid, kThreads, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(B), dA_cs, dtc,
        static_cast<float*>(states), p.L, (int)p.H, (int)p.G, (int)p.P, (int)p.N, p.Q, p.nc, p.ctab);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_scan_simt(const Plan& p, const void* x, const void* B, const void* C,
                                  const float* D, const float* dA_cs, const float* dtc,
                                  const void* states, void* y, hipStream_t s) {
  dim3 grid((unsigned)(p.nc * (p.Q / kIB) * p.batch * p.H));
  if (p.io == kBF16) {
    using T = __hip_bfloat16;
    chunk_scan_simt_kernel<T><<<grid, kThreads, 0, s>>>(
        static_cast<const T*>(x), static_cast<const T*>(B), static_cast<const T*>(C), D, dA_cs,
        dtc, static_cast<const T*>(states), static_cast<T*>(y), p.L, (int)p.H, (int)p.G,
        (int)p.P, (int)p.N, p.Q, p.nc, p.ctab);
  } else {
    chunk_scan_simt_kernel<float><<<grid, kThreads, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(B), static_cast<const float*>(C),
        D, dA_cs, dtc, static_cast<const float*>(states), static_cast<float*>(y), p.L, (int)p.H,
        (int)p.G, (int)p.P, (int)p.N, p.Q, p.nc, p.ctab);
  }
  return hipGetLastError();
}

}  // namespace ssd
