// Packed variable-length sequences: the per-chunk table every step reads in
// place of fixed-size chunks, and the per-sequence (first slot, chunk count)
// table that state passing walks, one chain per sequence and head.
//
// Sequence s holds tokens [cu[s], cu[s+1]) of the packed arrays. Its
// ceil(len/Q) chunks take consecutive table slots starting at the exclusive
// prefix sum of the chunk counts of the sequences before it; slots past the
// last sequence's chunks are marked unused (rows = 0). The recurrence restarts
// at the first chunk of every sequence, so no state crosses a boundary
// ("Mamba-2 vs Transformers: SSMs, structured state space duality", section
// "Practical integration notes ...": batched generation relies on padding
// conventions; packing the sequences avoids padding altogether).
//
// The offsets are sanitised on the device (clamped into [0, T] and to a
// non-negative length), and slots beyond the table are never written, so an
// invalid cu_seqlens can give wrong results but no out-of-range access.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kTabThreads = 1024;

__device__ __forceinline__ void seq_span(const int32_t* cu, int64_t s, int64_t T, int64_t& start, int64_t& len) {
  int64_t a = cu[s], e = cu[s + 1];
  a = a < 0 ? 0 : (a > T ? T : a);
  e = e < a ? a : (e > T ? T : e);
  start = a;
  len = e - a;
}

// One workgroup: a block-wide exclusive scan of the per-sequence chunk counts,
// 1024 sequences at a time, then each thread writes its sequence's slots.
__global__ __launch_bounds__(kTabThreads) void build_chunk_table_kernel(
    const int32_t* __restrict__ cu, int64_t S, int64_t T, int Q, int64_t nslots,
    ChunkInfo* __restrict__ tab, int2* __restrict__ seqtab) {
  __shared__ int64_t wsum[kTabThreads / 64];
  __shared__ int64_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < S; base += kTabThreads) {
    const int64_t s = base + tid;
    int64_t start = 0, len = 0;
    if (s < S) seq_span(cu, s, T, start, len);
    const int64_t n = (len + Q - 1) / Q;
    // inclusive scan inside the wavefront, then across wavefronts
    int64_t incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int64_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int64_t first = before + incl - n;
    if (s < S) {
      // slots past the table (only for invalid offsets) are dropped
      const int64_t fit = first >= nslots ? 0 : (first + n > nslots ? nslots - first : n);
      seqtab[s] = make_int2((int)(first < nslots ? first : 0), (int)fit);
    }
    for (int64_t k = 0; k < n; ++k) {
      const int64_t slot = first + k;
      if (slot >= nslots) break;
      const int64_t rows = len - k * Q < Q ? len - k * Q : Q;
      const int32_t flags = (k == 0 ? kFirstChunk : 0) | (k == n - 1 ? kLastChunk : 0);
      tab[slot] = ChunkInfo{(int32_t)(start + k * Q), (int32_t)rows, (int32_t)s, flags};
    }
    __syncthreads();
    if (tid == kTabThreads - 1) carry_s = before + incl;
    __syncthreads();
  }
  for (int64_t slot = carry_s + tid; slot < nslots; slot += kTabThreads)
    tab[slot] = ChunkInfo{0, 0, -1, 0};
}

}  // namespace

hipError_t launch_build_chunk_table(const int32_t* cu, int64_t S, int64_t T, int Q, int64_t nslots,
                                    ChunkInfo* tab, int2* seqtab, hipStream_t s) {
  build_chunk_table_kernel<<<1, kTabThreads, 0, s>>>(cu, S, T, Q, nslots, tab, seqtab);
  return hipGetLastError();
}

}  // namespace ssd
