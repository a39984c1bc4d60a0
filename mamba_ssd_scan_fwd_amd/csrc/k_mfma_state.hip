// Step 2 on bf16 matrix cores: the local state of every chunk,
//     S_c[p][n] = sum_{j in chunk c} w_j x_j[p] B_j[n],  w_j = exp(Lam_c - l_j) dt_j,
// i.e. the per-chunk SSM states that the blocked algorithm computes in
// parallel before recombining them ("Mamba-2 vs Transformers: SSMs,
// structured state space duality", section "Mamba-2 and the SSD paper: what
// changed in practice").
//
// As a matrix product per (b, c, h): S^T[N x P] = B_c^T[N x Q] * Xs[Q x P],
// with Xs = diag(w) x_c. The contraction runs over the chunk positions j and
// both operands are stored position-major in HBM (row j holds a contiguous P
// or N vector), so every 16-byte operand fragment of eight consecutive j is
// gathered from eight rows: tiles are transposed in registers (an 8x8 block
// per thread, eight coalesced 16-byte row reads) on their way into LDS.
//
// Work split: one workgroup (4 wavefronts) per (b, c, group of HB heads that
// share a B/C group, block of up to 128 state columns).
//  * B_c^T is staged through LDS once; each wavefront then keeps the
//    fragments of its own n tiles in registers for all HB heads, and the LDS
//    is reused as a double buffer for the scaled x of successive heads.
//  * LDS tiles are fragment-major (each lane's 16-byte fragment contiguous,
//    so operand reads are conflict-free) with a lane-slot swizzle that spreads
//    the staging writes over the banks.
//  * The x rows (and l, dt) of head hh+2 are loaded into one of two register
//    sets while head hh's products run; head hh+1's set is scaled by w_j,
//    rounded to bf16 and written transposed into the other LDS buffer; one
//    barrier per head.
//  * Output tiles hold four consecutive n per lane: 8-byte stores into
//    states[b,h,c][p][n].
#include "chunk_cumsum.h"
#include "mfma_common.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHB = 8;  // heads per workgroup, at most

template <int P, int NB, int Q>
struct StateCfg {
  static constexpr int NT_N = NB / 16, NT_P = P / 16;
  static constexpr int WN = NT_N >= 4 ? 4 : NT_N;  // wavefronts along n
  static constexpr int WP = 4 / WN;                // wavefronts along p
  static constexpr int TN = NT_N / WN;             // n tiles per wavefront
  static constexpr int TP = (NT_P + WP - 1) / WP;  // p tiles per wavefront
  static constexpr int KS = Q / 32;                // 32-deep steps over the chunk
  static constexpr int XBLK = (Q / 8) * (P / 8);   // 8x8 blocks of the x tile
  static constexpr int BBLK = (Q / 8) * (NB / 8);  // 8x8 blocks of the B tile
  static constexpr int XPT = (XBLK + kThreads - 1) / kThreads;
  static constexpr int BPT = (BBLK + kThreads - 1) / kThreads;
  static constexpr int X_FRAGS = NT_P * KS * 64;   // 16-byte fragments of one x buffer
  static constexpr int B_FRAGS = NT_N * KS * 64;
  static constexpr int LDS_FRAGS = (2 * X_FRAGS > B_FRAGS ? 2 * X_FRAGS : B_FRAGS);
  // fused cumsum: per head l and dt of the chunk, for up to kMaxHB heads
  static constexpr int TAB_FLOATS = kMaxHB * 2 * Q;
};

// slot of lane (r16, g4) inside a 1 KB fragment block (a bijection, so the
// matrix-core reads stay conflict-free; it spreads the transposed writes)
__device__ __forceinline__ int sslot(int r16, int g4, int tile) {
  return 16 * g4 + ((r16 + 2 * g4 + (tile & 1)) & 15);
}

// FUSED: the workgroup also computes the chunk's dA_cumsum and dt_chunked
// for its heads from dt and A (step 1), keeps them in LDS, and writes them to
// the workspace for the later steps (the workgroup of the first block of
// state columns does). Otherwise it reads them from dA_cs / dtc.
template <int P, int NB, int Q, bool FUSED>
__global__ __launch_bounds__(kThreads) void chunk_state_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ dA_cs, float* __restrict__ dtc,
    uint16_t* __restrict__ states, int64_t L, int H, int G, int N, int64_t nc, int HB, DtOpts dto,
    const ChunkInfo* __restrict__ ctab) {
  using C = StateCfg<P, NB, Q>;
  constexpr int KS = C::KS;
  constexpr int TAB_U4 = FUSED ? C::TAB_FLOATS / 4 : 0;
  __shared__ __align__(16) uint4 lds[C::LDS_FRAGS + TAB_U4];
  float* tab = reinterpret_cast<float*>(lds + C::LDS_FRAGS);  // [hh][l | dt][Q] (FUSED)

  const int nnb = N / NB;
  const int nhg = H / HB;
  int64_t bid = xcd_local_order(blockIdx.x, gridDim.x);
  const int nb = (int)(bid % nnb);
  bid /= nnb;
  const int hg = (int)(bid % nhg);
  bid /= nhg;
  const int64_t c = bid % nc;
  const int64_t b = bid / nc;
  const int h0 = hg * HB;
  const int g = h0 / (H / G);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int r16 = lane & 15, g4 = lane >> 4;
  int64_t row0;  // first token row of this chunk in the [batch * L] arrays
  int rows;      // valid positions in this chunk
  chunk_span(ctab, b, c, L, Q, row0, rows);
  if (rows <= 0) return;  // unused slot of a packed-sequence table (uniform)
  const int wn = wave % C::WN, wp = wave / C::WN;

  // ---- x of one head: raw rows into registers; scaled, transposed into LDS.
  // Two register sets: the loads of head hh+2 are issued while head hh's
  // products run, so about two heads of loads are in flight per workgroup. ----
  struct XSet {
    uint4 xr[C::XPT][8];
    float4 lr[C::XPT][2], dr[C::XPT][2];
    float lam;
  };
  auto fetch_x = [&](XSet& xs, int h) {
    if constexpr (!FUSED) {
      const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
      const float* dc = dtc + ((b * H + h) * nc + c) * Q;
      xs.lam = lc[Q - 1];
#pragma unroll
      for (int k = 0; k < C::XPT; ++k) {
        const int jb = ((tid + k * kThreads) / (P / 8)) % (Q / 8);
        xs.lr[k][0] = *reinterpret_cast<const float4*>(lc + 8 * jb);
        xs.lr[k][1] = *reinterpret_cast<const float4*>(lc + 8 * jb + 4);
        xs.dr[k][0] = *reinterpret_cast<const float4*>(dc + 8 * jb);
        xs.dr[k][1] = *reinterpret_cast<const float4*>(dc + 8 * jb + 4);
      }
    }
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * kThreads;
      const int cb = bi % (P / 8), jb = (bi / (P / 8)) % (Q / 8);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        // clamped row, always in bounds; rows past the end are zeroed later
        const int j = 8 * jb + rr;
        xs.xr[k][rr] = ld16(x + ((row0 + min(j, rows - 1)) * H + h) * P + 8 * cb);
      }
    }
  };
  auto stage_x = [&](XSet& xs, uint4* buf, int hh) {
    if constexpr (FUSED) {  // l and dt of this head from the LDS table
      const float* lt = tab + 2 * hh * Q;
      xs.lam = lt[Q - 1];
#pragma unroll
      for (int k = 0; k < C::XPT; ++k) {
        const int jb = ((tid + k * kThreads) / (P / 8)) % (Q / 8);
        xs.lr[k][0] = *reinterpret_cast<const float4*>(lt + 8 * jb);
        xs.lr[k][1] = *reinterpret_cast<const float4*>(lt + 8 * jb + 4);
        xs.dr[k][0] = *reinterpret_cast<const float4*>(lt + Q + 8 * jb);
        xs.dr[k][1] = *reinterpret_cast<const float4*>(lt + Q + 8 * jb + 4);
      }
    }
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * kThreads;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
        const float l8[8] = {xs.lr[k][0].x, xs.lr[k][0].y, xs.lr[k][0].z, xs.lr[k][0].w,
                             xs.lr[k][1].x, xs.lr[k][1].y, xs.lr[k][1].z, xs.lr[k][1].w};
        const float d8[8] = {xs.dr[k][0].x, xs.dr[k][0].y, xs.dr[k][0].z, xs.dr[k][0].w,
                             xs.dr[k][1].x, xs.dr[k][1].y, xs.dr[k][1].z, xs.dr[k][1].w};
        float w[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
          w[rr] = 8 * jb + rr < rows ? __expf(xs.lam - l8[rr]) * d8[rr] : 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {  // column p = 8cb + s: eight scaled bf16 along j
          uint32_t q[4];
#pragma unroll
          for (int m = 0; m < 4; ++m)
            q[m] = pack_bf16x2(w[2 * m] * bf16_at(xs.xr[k][2 * m], s),
                               w[2 * m + 1] * bf16_at(xs.xr[k][2 * m + 1], s));
          const int p = 8 * cb + s, pt = p >> 4;
          buf[(pt * KS + (jb >> 2)) * 64 + sslot(p & 15, jb & 3, pt)] = make_uint4(q[0], q[1], q[2], q[3]);
        }
      }
    }
  };

  // ---- prologue. All its global loads are issued first, in the order they
  // are consumed (dt, then B, then the x of the first two heads), so that each
  // wait covers one group only and the three latencies overlap. ----
  const int hlast = h0 + HB - 1;
  float dtv[kMaxHB];
  if constexpr (FUSED) {
    // dt of this chunk and these heads: a fixed count of loads (clamped)
    const float* drow = dt + (row0 + min(tid, rows - 1)) * H;
#pragma unroll
    for (int hh = 0; hh < kMaxHB; ++hh) dtv[hh] = drow[min(h0 + hh, hlast)];
  }
  uint4 braw[C::BPT][8];
#pragma unroll
  for (int k = 0; k < C::BPT; ++k) {
    const int bi = min(tid + k * kThreads, C::BBLK - 1);
    const int cb = bi % (NB / 8), jb = bi / (NB / 8);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int j = 8 * jb + rr;
      braw[k][rr] = ld16(Bm + ((row0 + min(j, rows - 1)) * G + g) * N + nb * NB + 8 * cb);
    }
  }
  XSet sa, sb;
  fetch_x(sa, h0);
  fetch_x(sb, min(h0 + 1, hlast));

  if constexpr (FUSED) {
    // ---- step 1 for this chunk and these heads: dt tile, then one
    // wavefront scan per head ----
    if (tid < Q) {
#pragma unroll
      for (int hh = 0; hh < kMaxHB; ++hh)
        if (hh < HB) tab[(2 * hh + 1) * Q + tid] = tid < rows ? dt_pre(dtv[hh], h0 + hh, dto) : 0.f;
    }
    __syncthreads();
    constexpr int QPL = Q / 64;
    for (int hh = wave; hh < HB; hh += kThreads / 64) {
      float d[QPL], sc[QPL];
#pragma unroll
      for (int k = 0; k < QPL; ++k) d[k] = tab[(2 * hh + 1) * Q + lane * QPL + k];
      wave_chunk_cumsum(d, A[h0 + hh], sc, lane);
#pragma unroll
      for (int k = 0; k < QPL; ++k) tab[2 * hh * Q + lane * QPL + k] = sc[k];
      if (nb == 0) {
        const int64_t base = ((b * H + h0 + hh) * nc + c) * Q + lane * QPL;
#pragma unroll
        for (int k = 0; k < QPL; ++k) {
          dA_cs[base + k] = sc[k];
          dtc[base + k] = d[k];
        }
      }
    }
    // the barrier after the B^T staging below also orders these LDS writes
  }

  // ---- B_c^T -> LDS fragments [nt][ks][slot] (once), then into registers ----
#pragma unroll
  for (int k = 0; k < C::BPT; ++k) {
    const int bi = tid + k * kThreads;
    if (bi < C::BBLK) {
      const int jb = bi / (NB / 8), cb = bi % (NB / 8);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)  // rows past the end are zero
        if (8 * jb + rr >= rows) braw[k][rr] = make_uint4(0, 0, 0, 0);
      uint4 o[8];
      transpose8x8(braw[k], o);
      // column n = 8cb + s holds B[8jb .. 8jb+7][n]: one fragment slot
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int n = 8 * cb + s, nt = n >> 4;
        lds[(nt * KS + (jb >> 2)) * 64 + sslot(n & 15, jb & 3, nt)] = o[s];
      }
    }
  }
  __syncthreads();
  bf16x8_t bt[C::TN][KS];
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
    const int nt = wn * C::TN + tn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bt[tn][ks] = as_bf16x8(lds[(nt * KS + ks) * 64 + sslot(r16, g4, nt)]);
  }
  __syncthreads();  // the LDS becomes the x double buffer

  stage_x(sa, lds, 0);
  __syncthreads();
  // head hh: its inputs are in LDS buffer hh & 1 (staged from `mine`, which
  // is refilled with head hh+2); `next` holds head hh+1, staged at the end.
  // The loads are always issued (the last heads re-read the final one), so
  // every head has the same memory-operation sequence.
  auto head = [&](XSet& mine, XSet& next, int hh) {
    const int h = h0 + hh;
    uint4* cur = lds + (hh & 1) * C::X_FRAGS;
    fetch_x(mine, min(h + 2, hlast));

    f32x4_t acc[C::TN][C::TP];
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int tp = 0; tp < C::TP; ++tp) acc[tn][tp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // all KS steps, also past the end of a ragged last chunk (its x rows are
    // zero there): straight-line code for the common full chunk
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t bb[C::TP];
#pragma unroll
      for (int tp = 0; tp < C::TP; ++tp) {
        const int pt = wp * C::TP + tp;
        // every p tile exists when the wavefronts split the p tiles evenly
        // (then this is no branch at all)
        bb[tp] = (C::WP * C::TP == C::NT_P || pt < C::NT_P)
                     ? as_bf16x8(cur[(pt * KS + ks) * 64 + sslot(r16, g4, pt)])
                     : as_bf16x8(make_uint4(0, 0, 0, 0));
      }
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
        for (int tp = 0; tp < C::TP; ++tp) acc[tn][tp] = mfma_16x16x32(bt[tn][ks], bb[tp], acc[tn][tp]);
    }

    // lane holds S^T[n = 4*g4 + i][p = r16] of each tile: four consecutive n
    uint16_t* out = states + ((b * H + h) * nc + c) * (int64_t)P * N;
#pragma unroll
    for (int tp = 0; tp < C::TP; ++tp) {
      const int pt = wp * C::TP + tp;
      if (C::WP * C::TP == C::NT_P || pt < C::NT_P) {
        const int p = pt * 16 + r16;
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
          const int n = nb * NB + (wn * C::TN + tn) * 16 + 4 * g4;
          const f32x4_t v = acc[tn][tp];
          *reinterpret_cast<uint2*>(out + (int64_t)p * N + n) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
    if (hh + 1 < HB) stage_x(next, lds + ((hh + 1) & 1) * C::X_FRAGS, hh + 1);  // the other buffer
    __syncthreads();
  };
  for (int hh = 0; hh < HB; hh += 2) {
    head(sa, sb, hh);
    if (hh + 1 < HB) head(sb, sa, hh + 1);
  }
}

// Heads per workgroup: a divisor of the heads in one B/C group, at most 8,
// as large as keeps the grid at >= 512 workgroups (two resident per compute
// unit; the B^T staging is amortised over more heads).
int pick_heads_per_wg(const Plan& p, int nnb) {
  const int64_t hpg = p.H / p.G;
  const int64_t base = p.batch * p.nc * nnb * p.H;
  int hb = 1;
  while (hb < kMaxHB && hpg % (hb * 2) == 0 && base / (hb * 2) >= 512) hb *= 2;
  return hb;
}

template <int P, int NB, int Q, bool FUSED>
hipError_t launch_pnq(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                      float* cs, float* dtc, void* st, hipStream_t s) {
  const int nnb = (int)(p.N / NB);
  const int hb = pick_heads_per_wg(p, nnb);
  const int64_t grid = p.batch * p.nc * (p.H / hb) * nnb;
  chunk_state_mfma_kernel<P, NB, Q, FUSED><<<dim3((unsigned)grid), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), dt, A, cs, dtc,
      static_cast<uint16_t*>(st), p.L, (int)p.H, (int)p.G, (int)p.N, p.nc, hb, p.dto, p.ctab);
  return hipGetLastError();
}

template <int P, int NB, bool FUSED>
hipError_t launch_pn(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                     float* cs, float* dtc, void* st, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_pnq<P, NB, 64, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 128: return launch_pnq<P, NB, 128, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 256: return launch_pnq<P, NB, 256, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    default: return hipErrorInvalidValue;
  }
}

template <int P, bool FUSED>
hipError_t launch_p(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                    float* cs, float* dtc, void* st, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_pn<P, 16, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 32: return launch_pn<P, 32, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 64: return launch_pn<P, 64, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    default: return launch_pn<P, 128, FUSED>(p, x, B, dt, A, cs, dtc, st, s);  // 128, 256
  }
}

template <bool FUSED>
hipError_t launch_any(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                      float* cs, float* dtc, void* st, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_p<16, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 32: return launch_p<32, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 64: return launch_p<64, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    case 128: return launch_p<128, FUSED>(p, x, B, dt, A, cs, dtc, st, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_chunk_state_supported(const Plan& p) {
  return p.io == kBF16 && (p.P == 16 || p.P == 32 || p.P == 64 || p.P == 128) &&
         (p.N == 16 || p.N == 32 || p.N == 64 || p.N == 128 || p.N == 256) &&
         (p.Q == 64 || p.Q == 128 || p.Q == 256);
}

hipError_t launch_chunk_state_mfma(const Plan& p, const void* x, const void* B,
                                   const float* dA_cs, const float* dtc, void* states,
                                   hipStream_t s) {
  return launch_any<false>(p, x, B, nullptr, nullptr, const_cast<float*>(dA_cs), const_cast<float*>(dtc),
                           states, s);
}

hipError_t launch_cumsum_chunk_state_mfma(const Plan& p, const void* x, const void* B, const float* dt,
                                          const float* A, float* dA_cs, float* dtc, void* states,
                                          hipStream_t s) {
  return launch_any<true>(p, x, B, dt, A, dA_cs, dtc, states, s);
}

}  // namespace ssd
