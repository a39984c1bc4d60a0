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
// or N vector), so every operand fragment of eight consecutive j is a column
// piece of a row-major tile.
//
// Work split: one workgroup (4 wavefronts) per (b, c, group of HB heads that
// share a B/C group, block of up to 128 state columns).
//  * The B tile goes straight from memory into the LDS in its natural row
//    order (loads that write the LDS directly; rows past the end of the chunk
//    read as zeros), and each wavefront reads the B_c^T fragments of its own
//    n tiles with the transposing LDS read, once, into registers kept for all
//    HB heads. The LDS is then reused as a double buffer for the scaled x of
//    successive heads.
//  * x has to be scaled by w_j before it is rounded to bf16, so it passes
//    through registers: the x rows (and l, dt) of head hh+1 are loaded into
//    registers while head hh's products run, then scaled, rounded and
//    written transposed (8x8 blocks) into the other LDS buffer,
//    fragment-major; one barrier per head. (Loading two heads ahead left the
//    last two heads' arithmetic with nothing in flight; one ahead is
//    slightly faster and frees a register set.) The slot permutation
//    inside each fragment block keeps both the staging writes and the
//    operand reads free of bank conflicts.
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
  static constexpr int XPT = (XBLK + kThreads - 1) / kThreads;
  // B tile: Q rows of NB bf16 in natural order (chunks swizzled per row),
  // loaded straight into the LDS in 1 KB blocks
  static constexpr int BRB = 2 * NB;
  static constexpr int BNBLK = Q * NB * 2 / 1024;
  static constexpr int BBPW = (BNBLK + kThreads / 64 - 1) / (kThreads / 64);
  static constexpr int X_FRAGS = NT_P * KS * 64;   // 16-byte fragments of one x buffer
  static constexpr int B_FRAGS = NT_N * KS * 64;
  static constexpr int LDS_FRAGS = (2 * X_FRAGS > B_FRAGS ? 2 * X_FRAGS : B_FRAGS);
  // fused cumsum: per head l and dt of the chunk, for up to kMaxHB heads
  static constexpr int TAB_FLOATS = kMaxHB * 2 * Q;
};

// Slot of lane (r, g) inside the 1 KB fragment block (pt, ks) of the scaled
// x tile: 16 g + (v & 15), v = r ^ (bit 3 of r) ^ (one constant per set bit
// of g and pt); a bijection per block. Measured on gfx950 (64 banks of 4
// bytes): a 16-byte read serves the eight-lane groups of a wavefront in the
// pairs (0-7, 24-31), (8-15, 16-23), (32-39, 56-63), (40-47, 48-55), each
// pair free of conflicts when its 16 lanes cover 256 bytes of distinct
// banks; a 16-byte write serves eight consecutive lanes over 128 bytes. Bit
// 3 of v follows bit 3 of r, which keeps every read pair on distinct banks;
// the other constants spread the eight threads of a staging write (eight
// columns p of 8x8 blocks: r = p % 16 with bit 3 from the column block,
// and the p tile) over the eight 16-byte positions.
template <int P>
__device__ __forceinline__ int xslot(int r, int g, int pt, int ks) {
  (void)ks;
  constexpr int mg0 = P == 16 || P == 32 ? 4 : 0;
  constexpr int mg1 = P == 16 ? 2 : 0;
  constexpr int mp0 = P == 16 ? 0 : 2;
  constexpr int mp1 = P >= 64 ? 4 : 0;
  const int v = r ^ ((r >> 3) & 1) ^ ((g & 1) ? mg0 : 0) ^ ((g & 2) ? mg1 : 0) ^ ((pt & 1) ? mp0 : 0) ^
                ((pt & 2) ? mp1 : 0);
  return 16 * g + (v & 15);
}
// Chunk permutation of B row j (NB bf16): the transposing 8-byte read of 16
// (32) lanes covers four (eight) rows at two adjacent chunks.
template <int NB>
__device__ __forceinline__ int bsw(int j) {
  return NB == 32 ? row_xor(j, 0, 2, 0, 2) : NB == 64 ? row_xor(j, 2, 4, 0, 2) : NB == 128 ? row_xor(j, 2, 4, 0, 8) : 0;
}

// MODE kReadCumsum: reads dA_cumsum and dt_chunked from dA_cs / dtc.
// MODE kFuseCumsum: the workgroup also computes the chunk's dA_cumsum and
// dt_chunked for its heads from dt and A (step 1), keeps them in LDS, and
// writes them to the workspace for the later steps (the workgroup of the
// first block of state columns does).
// MODE kWindowFinals: as kFuseCumsum over the end windows of packed
// sequences (ctab = the window table, slot c = sequence c), writing each
// sequence's fp32 final state to `fin` instead of a chunk state and no
// cumsum; for a window that continues a sequence from earlier chunks it adds
// the decayed state entering the window's chunk, read from hin ([H, hnc,
// P, N] bf16, the fixed chunks' entering states after state passing). An
// instantiation of its own, so the other modes keep their register budget.
constexpr int kReadCumsum = 0, kFuseCumsum = 1, kWindowFinals = 2;
template <int P, int NB, int Q, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_state_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ dA_cs, float* __restrict__ dtc,
    uint16_t* __restrict__ states, int64_t L, int H, int G, int N, int64_t nc, int HB, DtOpts dto,
    const ChunkInfo* __restrict__ ctab, const uint8_t* __restrict__ seg, float* __restrict__ fin,
    const uint16_t* __restrict__ hin, int64_t hnc) {
  using C = StateCfg<P, NB, Q>;
  constexpr bool FUSED = MODE != kReadCumsum;
  constexpr bool WIN = MODE == kWindowFinals;
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
  if (rows <= 0) {  // unused slot of a packed-sequence table (uniform)
    if constexpr (WIN) {  // the end window of an empty sequence: final state 0
      for (int hh = 0; hh < HB; ++hh) {
        float* o = fin + ((int64_t)c * H + h0 + hh) * (int64_t)P * N;
        for (int i = tid; i < P * NB / 4; i += kThreads) {
          const int p = i / (NB / 4), n = nb * NB + 4 * (i % (NB / 4));
          *reinterpret_cast<float4*>(o + (int64_t)p * N + n) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    return;
  }
  // end windows: the sequence started before the window (its final state
  // takes the decayed entering state)
  bool cross = false;
  if constexpr (WIN) cross = (ctab[c].flags & kWindowCrossing) != 0;
  const int wn = wave % C::WN, wp = wave / C::WN;

  // ---- x of one head: raw rows into registers; scaled, transposed into LDS.
  // The loads of head hh+1 are issued when head hh starts, so one head of
  // loads is in flight per workgroup while its products run. ----
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
      if (C::XPT * kThreads == C::XBLK || bi < C::XBLK) {  // (no branch when the blocks fill the threads)
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
          buf[(pt * KS + (jb >> 2)) * 64 + xslot<P>(p & 15, jb & 3, pt, jb >> 2)] = make_uint4(q[0], q[1], q[2], q[3]);
        }
      }
    }
  };

  // ---- prologue. All its global loads are issued first, in the order they
  // are consumed (dt, then B, then the x of the first head), so that each
  // wait covers one group only and the three latencies overlap. ----
  const int hlast = h0 + HB - 1;
  // B tile of the chunk straight into the LDS (rows past the end fall
  // outside the buffer range and arrive as zeros)
  {
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint4*)lds);
    const v4i32_t brs =
        buffer_words(Bm + (row0 * G + g) * N + nb * NB, (uint32_t)(((rows - 1) * (int64_t)G * N + NB) * 2));
#pragma unroll
    for (int k = 0; k < C::BBPW; ++k) {
      const int blk = wave * C::BBPW + k;
      if (blk < C::BNBLK) {
        const int pos = blk * 1024 + 16 * lane;
        const int j = pos / C::BRB, cp = (pos % C::BRB) / 16;
        dma16(brs, lds_base + blk * 1024, (uint32_t)(j * G * N * 2 + 16 * (cp ^ bsw<NB>(j))));
      }
    }
  }
  float dtv[kMaxHB];
  if constexpr (FUSED) {
    // dt of this chunk and these heads: a fixed count of loads (clamped)
    const float* drow = dt + (row0 + min(tid, rows - 1)) * H;
#pragma unroll
    for (int hh = 0; hh < kMaxHB; ++hh) dtv[hh] = drow[min(h0 + hh, hlast)];
  }
  XSet sa;
  fetch_x(sa, h0);

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
      if (seg != nullptr) {  // packed sequences in fixed chunks: the jumps at sequence starts
        bool st[QPL];
#pragma unroll
        for (int k = 0; k < QPL; ++k) {
          const int pos = lane * QPL + k;
          st[k] = pos < rows && seg[row0 + pos] != 0;
        }
        wave_chunk_cumsum_jump(d, A[h0 + hh], st, sc, lane);
      } else {
        wave_chunk_cumsum(d, A[h0 + hh], sc, lane);
      }
#pragma unroll
      for (int k = 0; k < QPL; ++k) tab[2 * hh * Q + lane * QPL + k] = sc[k];
      if (nb == 0 && !WIN) {
        const int64_t base = ((b * H + h0 + hh) * nc + c) * Q + lane * QPL;
#pragma unroll
        for (int k = 0; k < QPL; ++k) {
          dA_cs[base + k] = sc[k];
          dtc[base + k] = d[k];
        }
      }
    }
    // the barrier before the B^T reads below also orders these LDS writes
  }

  // ---- B_c^T fragments into registers (A operand, m = n, k = j): two
  // transposing reads each, lane (s, q) = (l % 16, l / 16) addressing row
  // 32 ks + 8 q + s / 4 (then 4 rows on), columns 16 nt + 4 (s % 4) .. +3,
  // so k runs over the eight consecutive j of the x fragments ----
  vm_wait<0>();
  __syncthreads();
  bf16x8_t bt[C::TN][KS];
  {
    const unsigned char* bl = reinterpret_cast<const unsigned char*>(lds);
    const int s = lane & 15, q = lane >> 4;
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int c2 = 2 * (wn * C::TN + tn) + ((s & 3) >> 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int j = 32 * ks + 8 * q + (s >> 2);
        const uint2 lo = lds_tr8(bl + j * C::BRB + 16 * (c2 ^ bsw<NB>(j)) + 8 * (s & 1));
        const uint2 hi = lds_tr8(bl + (j + 4) * C::BRB + 16 * (c2 ^ bsw<NB>(j + 4)) + 8 * (s & 1));
        bt[tn][ks] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
  }
  __syncthreads();  // the LDS becomes the x double buffer

  stage_x(sa, lds, 0);
  __syncthreads();
  // head hh: its inputs are in LDS buffer hh & 1; `mine` is refilled with
  // head hh+1 at the start and staged into the other buffer at the end. The
  // loads are always issued (the last head re-reads itself), so every head
  // has the same memory-operation sequence.
  auto head = [&](XSet& mine, int hh) {
    const int h = h0 + hh;
    uint4* cur = lds + (hh & 1) * C::X_FRAGS;
    fetch_x(mine, min(h + 1, hlast));
    // keep the loads here, issued before the products (the scheduler would
    // otherwise move them down next to their use and wait for them there)
    __builtin_amdgcn_sched_barrier(0);

    // end windows that continue a sequence: the entering state's four bf16
    // of each tile, loaded now so the loads overlap the products
    uint2 hv[C::TN][C::TP];
    if constexpr (WIN) {
      if (cross) {
        const uint16_t* hp = hin + ((int64_t)h * hnc + row0 / Q) * (int64_t)P * N;
#pragma unroll
        for (int tp = 0; tp < C::TP; ++tp) {
          const int pt = wp * C::TP + tp;
          if (C::WP * C::TP == C::NT_P || pt < C::NT_P) {
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) {
              const int n = nb * NB + (wn * C::TN + tn) * 16 + 4 * g4;
              hv[tn][tp] = *reinterpret_cast<const uint2*>(hp + (int64_t)(pt * 16 + r16) * N + n);
            }
          }
        }
      }
    }
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
                     ? as_bf16x8(cur[(pt * KS + ks) * 64 + xslot<P>(r16, g4, pt, ks)])
                     : as_bf16x8(make_uint4(0, 0, 0, 0));
      }
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
        for (int tp = 0; tp < C::TP; ++tp) acc[tn][tp] = mfma_16x16x32(bt[tn][ks], bb[tp], acc[tn][tp]);
    }

    // lane holds S^T[n = 4*g4 + i][p = r16] of each tile: four consecutive n
    if constexpr (WIN) {
      // end window of a packed sequence (batch 1, slot c = the sequence): its
      // final state in fp32, the window's state plus, for a sequence that
      // started earlier, exp(l at its last token) times the state entering
      // the chunk (the window then starts at the chunk's first row)
      const float carry = cross ? __expf(tab[2 * hh * Q + rows - 1]) : 0.f;
      float* o = fin + ((int64_t)c * H + h) * (int64_t)P * N;
#pragma unroll
      for (int tp = 0; tp < C::TP; ++tp) {
        const int pt = wp * C::TP + tp;
        if (C::WP * C::TP == C::NT_P || pt < C::NT_P) {
          const int p = pt * 16 + r16;
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            const int n = nb * NB + (wn * C::TN + tn) * 16 + 4 * g4;
            float4* q = reinterpret_cast<float4*>(o + (int64_t)p * N + n);
            f32x4_t v = acc[tn][tp];
            if (cross) {
              const uint2 t = hv[tn][tp];
              v[0] = fmaf(carry, __uint_as_float(t.x << 16), v[0]);
              v[1] = fmaf(carry, __uint_as_float(t.x & 0xffff0000u), v[1]);
              v[2] = fmaf(carry, __uint_as_float(t.y << 16), v[2]);
              v[3] = fmaf(carry, __uint_as_float(t.y & 0xffff0000u), v[3]);
            }
            *q = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
      stage_x(mine, lds + ((hh + 1) & 1) * C::X_FRAGS, hh + 1 < HB ? hh + 1 : hh);  // the other buffer
      __syncthreads();
      return;
    }
    uint16_t* out = states + ((b * H + h) * nc + c) * (int64_t)P * N;
#pragma unroll
    for (int tp = 0; tp < C::TP; ++tp) {
      const int pt = wp * C::TP + tp;
      if (C::WP * C::TP == C::NT_P || pt < C::NT_P) {
        const int p = pt * 16 + r16;
        if constexpr (C::TN % 2 == 0) {
          // two n tiles at a time: each lane stores eight consecutive n of
          // one row p (16 bytes), one store writing 64 contiguous bytes of
          // 16 rows
#pragma unroll
          for (int tn = 0; tn < C::TN; tn += 2) {
            const int n = nb * NB + (wn * C::TN + tn) * 16 + 16 * (g4 & 1) + 8 * (g4 >> 1);
            *reinterpret_cast<uint4*>(out + (int64_t)p * N + n) = pair_rows16(acc[tn][tp], acc[tn + 1][tp]);
          }
        } else {
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            const int n = nb * NB + (wn * C::TN + tn) * 16 + 4 * g4;
            const f32x4_t v = acc[tn][tp];
            *reinterpret_cast<uint2*>(out + (int64_t)p * N + n) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
        }
      }
    }
    // into the other buffer; also after the last head (its data again, never
    // read): staged unconditionally, the loads of `mine` have a use on every
    // path, which keeps them where they are issued, one head ahead, instead
    // of being sunk into a branch next to their use
    stage_x(mine, lds + ((hh + 1) & 1) * C::X_FRAGS, hh + 1 < HB ? hh + 1 : hh);
    __syncthreads();
  };
  for (int hh = 0; hh < HB; hh += 2) {
    head(sa, hh);
    if (hh + 1 < HB) head(sa, hh + 1);
  }
}

// Heads per workgroup: a divisor of the heads in one B/C group, at most 8,
// as large as keeps the grid at >= 512 workgroups (two resident per compute
// unit; the B^T staging is amortised over more heads). The end windows of
// packed sequences take the same rule: measured on the 32-sequence workload,
// grids of 1024 and 2048 smaller workgroups were 2% and 5% slower overall.
int pick_heads_per_wg(const Plan& p, int nnb) {
  const int64_t hpg = p.H / p.G;
  const int64_t base = p.batch * p.nc * nnb * p.H;
  int hb = 1;
  while (hb < kMaxHB && hpg % (hb * 2) == 0 && base / (hb * 2) >= 512) hb *= 2;
  return hb;
}

template <int P, int NB, int Q, int MODE>
hipError_t launch_pnq(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                      float* cs, float* dtc, void* st, hipStream_t s) {
  const int nnb = (int)(p.N / NB);
  const int hb = pick_heads_per_wg(p, nnb);
  const int64_t grid = p.batch * p.nc * (p.H / hb) * nnb;
  chunk_state_mfma_kernel<P, NB, Q, MODE><<<dim3((unsigned)grid), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), dt, A, cs, dtc,
      static_cast<uint16_t*>(st), p.L, (int)p.H, (int)p.G, (int)p.N, p.nc, hb, p.dto, p.ctab,
      MODE == kFuseCumsum ? p.seg_start : nullptr, MODE == kWindowFinals ? p.window_finals : nullptr,
      MODE == kWindowFinals ? static_cast<const uint16_t*>(p.window_hin) : nullptr, p.window_nc);
  return hipGetLastError();
}

template <int P, int NB, int MODE>
hipError_t launch_pn(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                     float* cs, float* dtc, void* st, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_pnq<P, NB, 64, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 128: return launch_pnq<P, NB, 128, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 256: return launch_pnq<P, NB, 256, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    default: return hipErrorInvalidValue;
  }
}

template <int P, int MODE>
hipError_t launch_p(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                    float* cs, float* dtc, void* st, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_pn<P, 16, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 32: return launch_pn<P, 32, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 64: return launch_pn<P, 64, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    default: return launch_pn<P, 128, MODE>(p, x, B, dt, A, cs, dtc, st, s);  // 128, 256
  }
}

template <int MODE>
hipError_t launch_any(const Plan& p, const void* x, const void* B, const float* dt, const float* A,
                      float* cs, float* dtc, void* st, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_p<16, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 32: return launch_p<32, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 64: return launch_p<64, MODE>(p, x, B, dt, A, cs, dtc, st, s);
    case 128: return launch_p<128, MODE>(p, x, B, dt, A, cs, dtc, st, s);
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
  return launch_any<kReadCumsum>(p, x, B, nullptr, nullptr, const_cast<float*>(dA_cs), const_cast<float*>(dtc),
                           states, s);
}

hipError_t launch_cumsum_chunk_state_mfma(const Plan& p, const void* x, const void* B, const float* dt,
                                          const float* A, float* dA_cs, float* dtc, void* states,
                                          hipStream_t s) {
  if (p.window_finals != nullptr) return launch_any<kWindowFinals>(p, x, B, dt, A, nullptr, nullptr, nullptr, s);
  return launch_any<kFuseCumsum>(p, x, B, dt, A, dA_cs, dtc, states, s);
}

}  // namespace ssd
