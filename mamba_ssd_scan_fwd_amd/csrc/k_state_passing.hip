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
    int64_t nc, int Q, int PN, int H, const int2* __restrict__ seqtab, uint32_t* __restrict__ stat,
    uint32_t tag) {
  const int64_t bh = blockIdx.x;
  if (stat != nullptr && bh == 0 && blockIdx.y == 0 && threadIdx.x == 0) {  // the forward's status record
    stat[0] = tag;
    stat[1] = 0u;
  }
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

  if (cnt <= 0) {  // an empty sequence: its final state is its initial state
    if (active && hT != nullptr) {
      float z[kVec];
      if (h0 != nullptr) {
        Vec8<float> v;
        v.load(h0 + bh * PN + e0);
        v.to(z);
      } else {
#pragma unroll
        for (int k = 0; k < kVec; ++k) z[k] = 0.f;
      }
      Vec8<float>::store(hT + bh * PN + e0, z);
    }
    return;
  }

  // Loads are issued from valid addresses only and not behind branches (a
  // branch join waits for the loads issued inside it, and a wait for the
  // newest load waits for all): an inactive thread reads element 0, a ring
  // slot past the chain's end re-reads its last chunk (never used).
  const int ec = active ? e0 : 0;
  const float* lam = dA_cs + (row * nc + c_beg) * Q + (Q - 1);
  // lane l's log-decay of chunk cb + l for the block of 64 chunks from cb;
  // the first block's is read before the ring's loads, so that waiting for
  // it drains nothing (later blocks' waits drain the ring once per 64)
  float lv = lam[(int64_t)(lane < cnt ? lane : cnt - 1) * Q];

  float h[kVec];
  {
    Vec8<float> v;
    v.load((h0 != nullptr ? h0 + bh * PN : dA_cs) + (h0 != nullptr ? ec : 0));
    float hv[kVec];
    v.to(hv);
#pragma unroll
    for (int k = 0; k < kVec; ++k) h[k] = h0 != nullptr && active ? hv[k] : 0.f;
  }

  TS* s = states + (row * nc + c_beg) * (int64_t)PN + ec;

  Vec8<TS> ring[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) ring[k].load(s + (int64_t)(k < cnt ? k : cnt - 1) * PN);

  for (int64_t cb = 0; cb < cnt; cb += 64) {
    const float dec = cb + lane < cnt ? __expf(lv) : 0.f;
    const int64_t ce = cb + 64 < cnt ? cb + 64 : cnt;
    for (int64_t c0 = cb; c0 < ce; c0 += PF) {
      // the PF steps run whole (c0 is a multiple of PF, which divides 64);
      // past the chain's end a step stores nothing and keeps h
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const int64_t c = c0 + k;
        const bool live = c < cnt;
        const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dec), (int)(c & 63)));
        float sv[kVec];
        ring[k].to(sv);
        ring[k].load(s + (c + PF < cnt ? c + PF : cnt - 1) * PN);
        if (live && active) Vec8<TS>::store(s + c * PN, h);
#pragma unroll
        for (int e = 0; e < kVec; ++e) h[e] = live ? fmaf(d, h[e], sv[e]) : h[e];
      }
    }
    const int64_t cn = cb + 64 + lane;  // the next block's
    lv = lam[(cn < cnt ? cn : cnt - 1) * Q];
  }
  if (active && hT != nullptr) Vec8<float>::store(hT + bh * PN + e0, h);
}

// Few long chains (a few long sequences): one chain step moves too few bytes
// for the whole GPU, so the chain's latency per step bounds the kernel above.
// Here each chain is cut into segments of KS chunks, one workgroup per
// (segment, chain, slice of 8 * kThreads state elements):
//  1. load the segment's KS chunk states (all loads in flight at once);
//  2. fold them from zero into the segment's aggregate A_s (fp32) and its
//     total log-decay, publish both and raise the segment's flag;
//  3. entering state of the segment: the initial state folded with the
//     aggregates of all earlier segments, H = exp(Lam_s') H + A_s' (waiting
//     for each flag);
//  4. walk the segment: Hin_c = H, H = exp(Lam_c) H + S_c; the last segment
//     writes the final state.
// A workgroup publishes before it waits, and takes a ticket at its start
// (segment-major), so every segment it waits for has started and publishes
// without waiting: no wait can block for good. Waits are bounded anyway (a
// status bit records one that was cut off). The initial state is read before
// publishing, so the last segment writes the final state only after every
// other workgroup has read the initial state (they may be the same buffer).
constexpr int kSegChunks = 32;
constexpr int kSpinLimit = 1 << 18;
constexpr uint32_t kCutOffBit = 2u;  // in the forward's status word (bit 0 is the one-pass kernel's)

template <typename TS, int KS>
__global__ __launch_bounds__(kThreads) void state_passing_seg_kernel(
    TS* __restrict__ states, const float* __restrict__ dA_cs, const float* h0, float* hT,
    float* __restrict__ agg, float* __restrict__ agg_lam, uint32_t* __restrict__ flags,
    uint32_t* __restrict__ ticket, uint32_t* __restrict__ status, int64_t nc, int Q, int PN, int64_t chains,
    int nslice, int nseg) {
  __shared__ uint32_t stk;
  if (threadIdx.x == 0) stk = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int64_t tk = __builtin_amdgcn_readfirstlane(stk);
  const int64_t per_seg = chains * nslice;
  if (tk >= per_seg * nseg) return;  // uniform
  const int seg = (int)(tk / per_seg);
  const int64_t bh = (tk - (int64_t)seg * per_seg) / nslice;
  const int slice = (int)(tk - (int64_t)seg * per_seg - bh * nslice);
  const int lane = threadIdx.x & 63;
  const int e0 = (slice * kThreads + threadIdx.x) * 8;
  const bool active = e0 < PN;
  const int64_t c_beg = (int64_t)seg * KS;
  const int cnt = (int)(nc - c_beg < KS ? nc - c_beg : KS);
  TS* s = states + (bh * nc + c_beg) * (int64_t)PN + e0;
  const float* lam = dA_cs + (bh * nc + c_beg) * Q + (Q - 1);

  // 1. the segment's chunk states, and lane l's exp(Lam) of chunk l
  Vec8<TS> sv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    if (active && k < cnt) sv[k].load(s + (int64_t)k * PN);
  const float lam_l = lane < cnt ? lam[(int64_t)lane * Q] : 0.f;
  const float dec_l = __expf(lam_l);
  float hin0[8];
  if (active && h0 != nullptr) {
    Vec8<float> v;
    v.load(h0 + bh * PN + e0);
    v.to(hin0);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) hin0[e] = 0.f;
  }

  // 2. aggregate and log-decay sum of the segment; publish them
  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    if (k < cnt) {
      const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dec_l), k));
      if (active) {
        float v[8];
        sv[k].to(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = fmaf(d, a[e], v[e]);
      }
    }
  }
  float lsum = lam_l;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
  if (seg + 1 < nseg) {
    if (active) {
      typedef int v4i __attribute__((ext_vector_type(4)));
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          agg + (bh * nseg + seg) * (int64_t)PN, 0, PN * 4, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(v4i{__float_as_int(a[0]), __float_as_int(a[1]), __float_as_int(a[2]), __float_as_int(a[3])}, r, e0 * 4, 0, 16 /* sc1 */);
      __builtin_amdgcn_raw_buffer_store_b128(v4i{__float_as_int(a[4]), __float_as_int(a[5]), __float_as_int(a[6]), __float_as_int(a[7])}, r, e0 * 4 + 16, 0, 16 /* sc1 */);
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(agg_lam + bh * nseg + seg, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(flags + (bh * nslice + slice) * nseg + seg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 3. the state entering the segment
  float h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = hin0[e];
  for (int sp = 0; sp < seg; ++sp) {
    const uint32_t* f = flags + (bh * nslice + slice) * nseg + sp;
    for (int spins = 0;; ++spins) {
      if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0) break;
      if (spins >= kSpinLimit) {
        if (lane == 0) __hip_atomic_fetch_or(status, kCutOffBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    asm volatile("" ::: "memory");  // the loads below stay after the flag
    const float dseg = __expf(__hip_atomic_load(agg_lam + bh * nseg + sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (active) {
      typedef int v4i __attribute__((ext_vector_type(4)));
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          agg + (bh * nseg + sp) * (int64_t)PN, 0, PN * 4, 0x00020000);
      const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, e0 * 4, 0, 16 /* sc1 */);
      const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(r, e0 * 4 + 16, 0, 16 /* sc1 */);
      const int av[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = fmaf(dseg, h[e], __int_as_float(av[e]));
    }
  }

  // 4. walk the segment
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    if (k < cnt) {
      const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dec_l), k));
      if (active) {
        float v[8];
        sv[k].to(v);
        Vec8<TS>::store(s + (int64_t)k * PN, h);
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = fmaf(d, h[e], v[e]);
      }
    }
  }
  if (seg + 1 == nseg && active && hT != nullptr) Vec8<float>::store(hT + bh * PN + e0, h);
}

__global__ void clear_words_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t* __restrict__ stat, uint32_t tag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
  if (stat != nullptr && i == 0) {
    stat[0] = tag;
    stat[1] = 0u;
  }
}

template <typename TS>
hipError_t launch_typed(const Plan& p, void* states, const float* dA_cs,
                        const float* h0, float* hT, uint32_t* stat, hipStream_t s) {
  const int PN = (int)(p.P * p.N);
  const int64_t chains = p.seqtab != nullptr ? p.nseq * p.H : p.batch * p.H;
  dim3 grid((unsigned)chains, (unsigned)((PN + kThreads * kVec - 1) / (kThreads * kVec)));
  state_passing_kernel<TS, 8><<<grid, kThreads, 0, s>>>(
      static_cast<TS*>(states), dA_cs, h0, hT, p.nc, p.Q, PN, (int)p.H, p.seqtab, stat, kPathSplit);
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_seg_typed(const Plan& p, void* states, const float* dA_cs, const float* h0, float* hT,
                            void* scratch, uint32_t* stat, bool cleared, hipStream_t s) {
  const int PN = (int)(p.P * p.N);
  const int64_t chains = p.batch * p.H;
  const int nslice = (PN + kThreads * kVec - 1) / (kThreads * kVec);
  const int nseg = (int)((p.nc + kSegChunks - 1) / kSegChunks);
  SegScratch sc = seg_scratch_layout(p, scratch);
  if (!cleared) {
    const int64_t nclear = sc.nwords;
    clear_words_kernel<<<dim3((unsigned)((nclear + 255) / 256)), 256, 0, s>>>(sc.flags, nclear, stat,
                                                                               kPathSplitSegmented);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t grid = chains * nslice * nseg;
  state_passing_seg_kernel<TS, kSegChunks><<<dim3((unsigned)grid), kThreads, 0, s>>>(
      static_cast<TS*>(states), dA_cs, h0, hT, sc.agg, sc.agg_lam, sc.flags, sc.ticket,
      stat != nullptr ? stat + 1 : sc.status, p.nc, p.Q, PN, chains, nslice, nseg);
  return hipGetLastError();
}

}  // namespace

// Host-only: the segmented kernel serves batched layouts whose chains are too
// few to fill the GPU with the plain kernel (under 512 of its workgroups) and
// long enough to cut (at least two segments). Each segment folds in every
// earlier segment's aggregate, so the aggregate reads grow with the square of
// the segment count: at most 32 segments (1024 chunks) take this path.
constexpr int64_t kMaxSegs = 32;
bool seg_state_passing_applies(const Plan& p) {
  if (p.seqtab != nullptr || p.nc < 2 * kSegChunks || p.nc > kMaxSegs * kSegChunks) return false;
  const int64_t PN = p.P * p.N;
  const int64_t nslice = (PN + kThreads * kVec - 1) / (kThreads * kVec);
  return p.batch * p.H * nslice < 512;
}

// [aggregates: chains * nseg * PN fp32][log-decay sums: chains * nseg fp32]
// [flags: chains * nslice * nseg][ticket][status] (32-bit words, cleared by
// the launch), each part on a 256-byte boundary.
SegScratch seg_scratch_layout(const Plan& p, void* base) {
  const int64_t PN = p.P * p.N;
  const int64_t chains = p.batch * p.H;
  const int64_t nslice = (PN + kThreads * kVec - 1) / (kThreads * kVec);
  const int64_t nseg = (p.nc + kSegChunks - 1) / kSegChunks;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t agg_b = up(size_t(chains * nseg * PN) * 4);
  const size_t lam_b = up(size_t(chains * nseg) * 4);
  SegScratch sc;
  sc.nwords = chains * nslice * nseg + 2;
  sc.chains = chains;
  sc.nslice = nslice;
  sc.nseg = nseg;
  sc.bytes = agg_b + lam_b + up(size_t(sc.nwords) * 4);
  char* b = static_cast<char*>(base);
  sc.agg = reinterpret_cast<float*>(b);
  sc.agg_lam = reinterpret_cast<float*>(b + agg_b);
  sc.flags = reinterpret_cast<uint32_t*>(b + agg_b + lam_b);
  sc.ticket = sc.flags + chains * nslice * nseg;
  sc.status = sc.ticket + 1;
  return sc;
}

hipError_t launch_state_passing_seg(const Plan& p, void* states, const float* dA_cs, const float* h0, float* hT,
                                    void* scratch, uint32_t* stat, hipStream_t s, bool cleared) {
  if (p.io == kBF16) return launch_seg_typed<__hip_bfloat16>(p, states, dA_cs, h0, hT, scratch, stat, cleared, s);
  return launch_seg_typed<float>(p, states, dA_cs, h0, hT, scratch, stat, cleared, s);
}

hipError_t launch_state_passing(const Plan& p, void* states, const float* dA_cs,
                                const float* h0, float* hT, hipStream_t s, uint32_t* stat) {
  if (p.io == kBF16) return launch_typed<__hip_bfloat16>(p, states, dA_cs, h0, hT, stat, s);
  return launch_typed<float>(p, states, dA_cs, h0, hT, stat, s);
}

int64_t seg_state_passing_grid(const Plan& p) {
  const int64_t PN = p.P * p.N;
  const int64_t nslice = (PN + kThreads * kVec - 1) / (kThreads * kVec);
  return p.batch * p.H * nslice * ((p.nc + kSegChunks - 1) / kSegChunks);
}

}  // namespace ssd
