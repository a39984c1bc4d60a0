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

// ---- packed sequences in fixed chunks -------------------------------------
//
// Without initial states the packed stream is cut into the fixed Q-token
// chunks of one long sequence, and every sequence start enters the chunk
// cumsum as a jump of -kSegJump (chunk_cumsum.h): every decay across a start
// is then exactly 0, so the chunk-state, state-passing and chunk-scan steps
// run unchanged and keep each sequence to itself. A chunk may hold the end of
// one sequence and the start of the next; no chunk is partial except the
// last of the stream.
//
// The final state of sequence s is the state after its last token e. Its end
// window runs from the start of the chunk holding e to e; the window's local
// state (the chunk-state step on the window, with the same jumps) plus the
// state entering that chunk times exp(l'_e) (the window's cumsum at e: 0 when
// the sequence starts inside the window) is the final state.

__device__ __forceinline__ int64_t clamped_start(const int32_t* cu, int64_t s, int64_t T) {
  const int64_t a = cu[s];
  return a < 0 ? 0 : (a > T ? T : a);
}

// seg_start[t] = 1 where a non-empty sequence starts after token 0 (nothing
// precedes token 0, so no decay has to be cut there). wtab[s] = the end
// window of sequence s: from the later of its first token and its last
// token's chunk start, to its last token (rows 0 for an empty sequence), so
// it holds tokens of s only; flags kWindowCrossing when s started in an
// earlier chunk. Also zeroes clear[0, nclear) and writes the status record.
__device__ __forceinline__ int64_t seq_holding(const int32_t* cu, int64_t S, int64_t T, int64_t t) {
  // the last sequence whose start is <= t: with valid offsets, the non-empty
  // sequence that holds t (an empty one starts where the next one does)
  int64_t lo = 0, hi = S - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (clamped_start(cu, mid, T) <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void build_packed_tables_kernel(const int32_t* __restrict__ cu, int64_t S,
                                                                  int64_t T, int Q, uint8_t* __restrict__ seg_start,
                                                                  ChunkInfo* __restrict__ wtab,
                                                                  uint32_t* __restrict__ clear, int64_t nclear,
                                                                  uint32_t* __restrict__ stat, uint32_t tag) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (stat != nullptr && i0 == 0) {
    stat[0] = tag;
    stat[1] = 0u;
  }
  for (int64_t i = i0; i < nclear; i += stride) clear[i] = 0u;
  for (int64_t t = i0; t < T; t += stride)
    seg_start[t] = t > 0 && clamped_start(cu, seq_holding(cu, S, T, t), T) == t ? 1 : 0;
  for (int64_t s = i0; s < S; s += stride) {
    int64_t start, len;
    seq_span(cu, s, T, start, len);
    if (len == 0) {
      wtab[s] = ChunkInfo{0, 0, (int32_t)s, 0};
    } else {
      const int64_t e = start + len - 1;
      const int64_t c0 = e / Q * Q;
      const int64_t t0 = start > c0 ? start : c0;
      wtab[s] = ChunkInfo{(int32_t)t0, (int32_t)(e - t0 + 1), (int32_t)s, start < c0 ? kWindowCrossing : 0};
    }
  }
}

}  // namespace

hipError_t launch_build_packed_tables(const int32_t* cu, int64_t S, int64_t T, int Q, uint8_t* seg_start,
                                      ChunkInfo* wtab, uint32_t* clear, int64_t nclear, uint32_t* stat,
                                      uint32_t tag, hipStream_t s) {
  int64_t work = T > S ? T : S;
  if (nclear > work) work = nclear;
  const int64_t blocks = (work + 255) / 256 < 4096 ? (work + 255) / 256 : 4096;
  build_packed_tables_kernel<<<dim3((unsigned)(blocks > 0 ? blocks : 1)), 256, 0, s>>>(cu, S, T, Q, seg_start, wtab,
                                                                                     clear, nclear, stat, tag);
  return hipGetLastError();
}

hipError_t launch_build_chunk_table(const int32_t* cu, int64_t S, int64_t T, int Q, int64_t nslots,
                                    ChunkInfo* tab, int2* seqtab, hipStream_t s) {
  build_chunk_table_kernel<<<1, kTabThreads, 0, s>>>(cu, S, T, Q, nslots, tab, seqtab);
  return hipGetLastError();
}

}  // namespace ssd
