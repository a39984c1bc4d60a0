// Step 1: per-chunk inclusive cumulative sum of dt * A.
//
// The blocked algorithm processes the sequence in chunks ("Mamba-2 vs
// Transformers: SSMs, structured state space duality", section "Mamba-2 and
// the SSD paper: what changed in practice"); inside chunk c the decay between
// positions j <= i is exp(l_i - l_j) with l the inclusive sum of dt*A from the
// chunk start. This kernel produces l (dA_cumsum) and dt regrouped per chunk
// (dt_chunked), both [batch, H, nc, Q] fp32 with the positions of a chunk
// contiguous, so the contraction kernels read one contiguous run per
// (b, h, c). Positions past the sequence end get dt = 0, so l stays flat.
//
// Mapping: one workgroup per (chunk, batch, block of HB heads) with one
// wavefront per head. The dt tile [Q][HB] is read with the head index fastest
// (coalesced along dt's innermost axis) into LDS; then each wavefront scans
// its head's Q positions: each lane owns Q/64 consecutive positions, scans
// them serially, and the lane totals are combined with a log-step wavefront
// scan (__shfl_up).
// Optionally the launch also sets a run of 32-bit words to zero (the
// counters the one-pass kernel that follows synchronises on) and records the
// forward path in a status record of the workspace (path tag, status bits
// cleared).
#include "chunk_cumsum.h"

namespace ssd {
namespace {

constexpr int kHB = 16;             // heads per workgroup
constexpr int kThreads = 64 * kHB;  // one wavefront per head

template <int Q>
__global__ __launch_bounds__(kThreads) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ dA_cs, float* __restrict__ dtc,
    int64_t L, int H, int64_t nc, DtOpts dto, const ChunkInfo* __restrict__ ctab,
    const uint8_t* __restrict__ seg, uint32_t* __restrict__ clear, int64_t nclear,
    uint32_t* __restrict__ stat, uint32_t tag) {
  constexpr int QPL = Q / 64;  // positions per lane
  __shared__ float tile[Q][kHB + 1];
  const int64_t c = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int h0 = blockIdx.z * kHB;
  const int hb = min(kHB, H - h0);
  const int tid = threadIdx.x;
  if (clear != nullptr) {
    const int64_t nthreads = int64_t(gridDim.x) * gridDim.y * gridDim.z * kThreads;
    const int64_t gid = ((int64_t(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * kThreads + tid;
    for (int64_t i = gid; i < nclear; i += nthreads) clear[i] = 0u;
  }
  if (stat != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) {
    stat[0] = tag;
    stat[1] = 0u;
  }

  int64_t row0;
  int rows;
  chunk_span(ctab, b, c, L, Q, row0, rows);
  for (int idx = tid; idx < Q * kHB; idx += kThreads) {
    const int i = idx / kHB, hh = idx % kHB;
    float v = 0.f;
    if (hh < hb && i < rows) v = dt_pre(dt[(row0 + i) * H + h0 + hh], h0 + hh, dto);
    tile[i][hh] = v;
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int hh = wave; hh < hb; hh += kThreads / 64) {
    const int h = h0 + hh;
    const float a = A[h];
    float d[QPL], s[QPL];
#pragma unroll
    for (int k = 0; k < QPL; ++k) d[k] = tile[lane * QPL + k][hh];
    if (seg != nullptr) {  // packed sequences in fixed chunks: the jumps at sequence starts
      bool st[QPL];
#pragma unroll
      for (int k = 0; k < QPL; ++k) {
        const int pos = lane * QPL + k;
        st[k] = pos < rows && seg[row0 + pos] != 0;
      }
      wave_chunk_cumsum_jump(d, a, st, s, lane);
    } else {
      wave_chunk_cumsum(d, a, s, lane);
    }
    const int64_t base = (((b * H + h) * nc) + c) * Q + lane * QPL;
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      dA_cs[base + k] = s[k];
      dtc[base + k] = d[k];
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum_clear(const Plan& p, const float* dt, const float* A, float* dA_cs, float* dtc,
                                     uint32_t* clear, int64_t nclear, uint32_t* stat, uint32_t tag,
                                     hipStream_t s) {
  dim3 grid((unsigned)p.nc, (unsigned)p.batch, (unsigned)((p.H + kHB - 1) / kHB));
  switch (p.Q) {
    case 64:
      chunk_cumsum_kernel<64><<<grid, kThreads, 0, s>>>(dt, A, dA_cs, dtc, p.L, (int)p.H, p.nc, p.dto, p.ctab, p.seg_start, clear,
                                                        nclear, stat, tag);
      break;
    case 128:
      chunk_cumsum_kernel<128><<<grid, kThreads, 0, s>>>(dt, A, dA_cs, dtc, p.L, (int)p.H, p.nc, p.dto, p.ctab, p.seg_start, clear,
                                                         nclear, stat, tag);
      break;
    case 256:
      chunk_cumsum_kernel<256><<<grid, kThreads, 0, s>>>(dt, A, dA_cs, dtc, p.L, (int)p.H, p.nc, p.dto, p.ctab, p.seg_start, clear,
                                                         nclear, stat, tag);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_chunk_cumsum(const Plan& p, const float* dt, const float* A,
                               float* dA_cs, float* dtc, hipStream_t s) {
  return launch_chunk_cumsum_clear(p, dt, A, dA_cs, dtc, nullptr, 0, nullptr, 0, s);
}

}  // namespace ssd
