// Internal declarations shared by the host planner (api.cpp) and the kernel
// translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <cstdint>

namespace ssd {

enum IoType : int { kF32 = 0, kBF16 = 1 };

// dt preprocessing (bias, softplus, clamp) as the descriptor asks for it.
struct DtOpts {
  const float* bias;  // [H] or nullptr
  int softplus, clamp;
  float lo, hi;
};

// Where chunk c lies when sequences are packed (variable lengths): tokens
// [t0, t0 + rows) of the packed [T, ...] arrays, sequence `seq`, and flags
// kFirstChunk / kLastChunk of that sequence. rows == 0 marks an unused slot.
struct ChunkInfo {
  int32_t t0, rows, seq, flags;
};
constexpr int32_t kFirstChunk = 1, kLastChunk = 2;
// End windows of packed sequences in fixed chunks (one slot per sequence:
// from the later of its first token and its last token's chunk start, to its
// last token): the sequence started in an earlier chunk, so its final state
// takes the decayed state entering the window's chunk.
constexpr int32_t kWindowCrossing = 4;
// The chunk count of a sequence is also kept per sequence (first slot, count)
// so that state passing can run one chain per sequence.

// A validated problem plus the chosen chunk length.
struct Plan {
  DtOpts dto;
  const ChunkInfo* ctab = nullptr;  // packed sequences: per-chunk table (device), else null
  const int2* seqtab = nullptr;     // packed sequences: (first slot, chunk count) per sequence
  int64_t nseq = 0;                 // packed sequences: their number
  // packed sequences in fixed chunks: 1 at every token where a sequence
  // starts (the cumsum's jumps, kSegJump), else nullptr
  const uint8_t* seg_start = nullptr;
  // end windows of packed sequences (ctab = the window table, nc = S, batch
  // 1): the chunk-state kernel writes each sequence's fp32 final state here
  // ([S, H, P, N]) instead of chunk states, taking the states entering the
  // fixed chunks (bf16 [H, window_nc, P, N], after state passing) from
  // window_hin
  float* window_finals = nullptr;
  const void* window_hin = nullptr;
  int64_t window_nc = 0;
  int64_t batch, L, H, P, N, G;
  int io;       // IoType of x, B, C, y and of the chunk states
  int Q;        // chunk length
  int64_t nc;   // number of chunks = ceil(L / Q)
  int64_t heads_per_group() const { return H / G; }
  size_t io_bytes() const { return io == kBF16 ? 2 : 4; }
};

// The status record a whole-forward call leaves in its workspace: word 0 the
// path it took (tags below, written by its first kernel that runs on every
// path), word 1 the status bits (cleared by that same kernel; a bounded wait
// that gives up ORs its bit in).
constexpr uint32_t kPathSplit = 1, kPathSplitSegmented = 2, kPathOnePass = 3;

// Step launchers. Each returns the hipGetLastError() after its launches.
hipError_t launch_chunk_cumsum(const Plan& p, const float* dt, const float* A,
                               float* dA_cs, float* dtc, hipStream_t s);
hipError_t launch_chunk_state(const Plan& p, const void* x, const void* B,
                              const float* dA_cs, const float* dtc, void* states,
                              hipStream_t s);
// stat: the forward's status record (nullptr for the step entry point and
// packed sequences), tagged kPathSplit.
hipError_t launch_state_passing(const Plan& p, void* states, const float* dA_cs,
                                const float* h0, float* hT, hipStream_t s, uint32_t* stat = nullptr);
// State passing for a few long chains: segments of one chain in parallel,
// with scratch from the workspace (seg_scratch_layout(p, nullptr).bytes).
struct SegScratch {
  float* agg;
  float* agg_lam;
  uint32_t* flags;  // then the ticket and the status word
  uint32_t* ticket;
  uint32_t* status;
  int64_t nwords;   // flags + ticket + status
  int64_t chains, nslice, nseg;  // flags[(chain * nslice + slice) * nseg + segment]
  size_t bytes;
};
bool seg_state_passing_applies(const Plan& p);
SegScratch seg_scratch_layout(const Plan& p, void* base);
// stat: the forward's status record, tagged kPathSplitSegmented; a cut-off
// wait sets bit 1 of its status word.
// cleared: the scratch's flags, ticket and status words are already zero and
// the record written (by an earlier kernel on the stream), so the launch
// skips its clearing kernel.
hipError_t launch_state_passing_seg(const Plan& p, void* states, const float* dA_cs, const float* h0, float* hT,
                                    void* scratch, uint32_t* stat, hipStream_t s, bool cleared = false);
int64_t seg_state_passing_grid(const Plan& p);  // workgroups (= tickets) of one launch
hipError_t launch_chunk_scan(const Plan& p, const void* x, const void* B, const void* C,
                             const float* D, const float* dA_cs, const float* dtc,
                             const void* states, void* y, hipStream_t s);

// Steps 1 to 5 on the one-pass path: the cumsum launch (which also clears
// the words the chain synchronises on) and the fused state/output kernel.
struct FusedArgs {
  const void* x;
  const void* B;
  const void* C;
  const float* D;
  const float* dA_cs;
  const float* dtc;
  const float* h_init;  // [batch, H, P, N] fp32 or nullptr (zeros)
  void* y;
  float* h_final;       // [batch, H, P, N] fp32 or nullptr
  float* ring;          // [batch, H, 2, P * N] fp32 hand-over slots
  uint32_t* flags;      // [batch * H] per-head chunk counters, zero at launch
  uint32_t* ticket;     // workgroup ticket counter, zero at launch
  uint32_t* status;     // the status record's word 1: bit 0 set when a wait for a state was cut off
};
bool fused_forward_supported(const Plan& p);
bool fused_forward_preferred(const Plan& p);  // supported and measured faster than the split path
size_t fused_ring_bytes(const Plan& p);
int64_t fused_forward_grid(const Plan& p);  // workgroups (= tickets) of one launch
// The cumsum, also setting words [clear, clear + nclear) to zero and, when
// stat != nullptr, writing the status record {tag, 0}.
hipError_t launch_chunk_cumsum_clear(const Plan& p, const float* dt, const float* A, float* dA_cs, float* dtc,
                                     uint32_t* clear, int64_t nclear, uint32_t* stat, uint32_t tag,
                                     hipStream_t s);
hipError_t launch_fused_forward(const Plan& p, const FusedArgs& a, hipStream_t s);

// Packed sequences in fixed chunks (k_varlen.hip): the per-token sequence
// start flags and, per sequence, its end window (from the start of the chunk
// holding its last token to that token); then each sequence's final state
// from its window's local state and the state entering the window's chunk.
// Also zeroes clear[0, nclear) and, when stat is given, writes the status
// record {tag, 0}.
hipError_t launch_build_packed_tables(const int32_t* cu, int64_t S, int64_t T, int Q, uint8_t* seg_start,
                                      ChunkInfo* wtab, uint32_t* clear, int64_t nclear, uint32_t* stat,
                                      uint32_t tag, hipStream_t s);

hipError_t launch_conv1d_split(const Plan& p, int K, const void* xbc, const float* w, const float* bias, int act,
                               const float* st_in, float* st_out, void* x, void* B, void* C, hipStream_t s);
hipError_t launch_decode_step(const Plan& p, const void* x, const float* dt, const float* A, const void* B,
                              const void* C, const float* D, float* state, void* y, hipStream_t s);

// Compute units of the current device (queried once per device).
int device_cu_count();

// First row (of the [batch * L, ...] token arrays) and valid length of chunk
// c of batch b: fixed-size chunks of each sequence, or the packed table.
__device__ __forceinline__ void chunk_span(const ChunkInfo* tab, int64_t b, int64_t c, int64_t L, int Q,
                                           int64_t& row0, int& rows) {
  if (tab != nullptr) {
    const ChunkInfo ci = tab[c];
    row0 = ci.t0;
    rows = ci.rows;
  } else {
    row0 = b * L + c * Q;
    rows = (int)(L - c * Q < Q ? L - c * Q : Q);
  }
}

// Element conversion helpers used by every kernel file.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__hip_bfloat16 v) { return __bfloat162float(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __hip_bfloat16 from_f32<__hip_bfloat16>(float v) {
  return __float2bfloat16(v);  // round to nearest even
}

}  // namespace ssd
