// Step 2 on bf16 matrix cores: the local state of every chunk,
//     S_c[p][n] = sum_{j in chunk c} w_j x_j[p] B_j[n],  w_j = exp(Lam_c - l_j) dt_j,
// i.e. the per-chunk SSM states that the blocked algorithm computes in
// parallel before recombining them ("Mamba-2 vs Transformers: SSMs,
// structured state space duality", section "Mamba-2 and the SSD paper: what
// changed in practice").
//
// As a matrix product per (b, c, h): S^T[N x P] = B_c^T[N x Q] * Xs[Q x P],
// with Xs = diag(w) x_c. The contraction runs over the chunk positions j, and
// both operands are stored position-major in HBM (row j holds a contiguous P
// or N vector), so each 16-byte operand fragment of eight consecutive j must
// be gathered from eight rows. Tiles are therefore staged through LDS
// transposed ([n][j] and [p][j], j contiguous): every thread loads an 8x8
// block with eight coalesced 16-byte row reads, transposes it in registers
// (x is scaled by w_j and rounded to bf16 on the way), and writes eight
// 16-byte LDS rows; the matrix-core loop then reads each fragment with one
// 16-byte LDS read.
//
// Work split: one workgroup (4 wavefronts) per (b, c, group of HB heads that
// share a B/C group, block of up to 128 state columns). B_c^T is staged once
// and reused by the HB heads; the next head's x block is loaded into
// registers while the current head's products run. Output tiles hold four
// consecutive n per lane, written as 8-byte stores into states[b,h,c][p][n].
#include "mfma_common.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

template <int P, int NB, int Q>
struct StateCfg {
  static constexpr int QP = Q + 8;  // LDS row pitch (bf16): 16-byte pad spreads banks
  static constexpr int NT_N = NB / 16, NT_P = P / 16;
  static constexpr int WN = NT_N >= 4 ? 4 : NT_N;  // wavefronts along n
  static constexpr int WP = 4 / WN;                // wavefronts along p
  static constexpr int TN = NT_N / WN;             // n tiles per wavefront
  static constexpr int TP = (NT_P + WP - 1) / WP;  // p tiles per wavefront
  static constexpr int XBLK = (Q / 8) * (P / 8);   // 8x8 blocks in the x tile
  static constexpr int BBLK = (Q / 8) * (NB / 8);  // 8x8 blocks in the B tile
  static constexpr int XPT = (XBLK + kThreads - 1) / kThreads;
  static constexpr int BPT = (BBLK + kThreads - 1) / kThreads;
  static constexpr size_t lds_bytes = size_t(NB + P) * QP * 2;
};

template <int P, int NB, int Q>
__global__ __launch_bounds__(kThreads) void chunk_state_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const float* __restrict__ dA_cs, const float* __restrict__ dtc,
    uint16_t* __restrict__ states, int64_t L, int H, int G, int N, int64_t nc, int HB) {
  using C = StateCfg<P, NB, Q>;
  __shared__ __align__(16) uint16_t sB[NB * C::QP];
  __shared__ __align__(16) uint16_t sX[P * C::QP];

  const int nnb = N / NB;
  const int nhg = H / HB;
  int64_t bid = blockIdx.x;
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
  const int64_t t0 = c * Q;
  const int rows = (int)(L - t0 < Q ? L - t0 : Q);  // valid positions in this chunk

  // ---- B_c^T -> sB[n][j] (once per workgroup) ----
#pragma unroll
  for (int k = 0; k < C::BPT; ++k) {
    const int bi = tid + k * kThreads;
    if (bi < C::BBLK) {
      const int cb = bi % (NB / 8), jb = bi / (NB / 8);
      uint4 r[8], o[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int j = 8 * jb + rr;
        r[rr] = ld16_keep(Bm + ((b * L + t0 + min(j, rows - 1)) * G + g) * N + nb * NB + 8 * cb, j < rows);
      }
      transpose8x8(r, o);
#pragma unroll
      for (int s = 0; s < 8; ++s) st16(sB + (8 * cb + s) * C::QP + 8 * jb, o[s]);
    }
  }

  // ---- x block loader: thread block bi covers rows 8jb..8jb+7, cols 8cb..8cb+7 ----
  uint4 xr[C::XPT][8];
  float4 lr[C::XPT][2], dr[C::XPT][2];
  float lam = 0.f;
  auto load_x = [&](int h) {
    const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
    const float* dc = dtc + ((b * H + h) * nc + c) * Q;
    lam = lc[Q - 1];
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * kThreads;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int j = 8 * jb + rr;
          // raw load (clamped row, always in bounds): rows past the end are
          // zeroed when staged, so nothing here waits for the data
          xr[k][rr] = ld16(x + ((b * L + t0 + min(j, rows - 1)) * H + h) * P + 8 * cb);
        }
        lr[k][0] = *reinterpret_cast<const float4*>(lc + 8 * jb);
        lr[k][1] = *reinterpret_cast<const float4*>(lc + 8 * jb + 4);
        dr[k][0] = *reinterpret_cast<const float4*>(dc + 8 * jb);
        dr[k][1] = *reinterpret_cast<const float4*>(dc + 8 * jb + 4);
      }
    }
  };
  // scale rows by w_j = exp(Lam - l_j) dt_j, round to bf16, write transposed
  auto store_x = [&]() {
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * kThreads;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
        const float l8[8] = {lr[k][0].x, lr[k][0].y, lr[k][0].z, lr[k][0].w,
                             lr[k][1].x, lr[k][1].y, lr[k][1].z, lr[k][1].w};
        const float d8[8] = {dr[k][0].x, dr[k][0].y, dr[k][0].z, dr[k][0].w,
                             dr[k][1].x, dr[k][1].y, dr[k][1].z, dr[k][1].w};
        float w[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          w[rr] = __expf(lam - l8[rr]) * d8[rr];
          if (8 * jb + rr >= rows) xr[k][rr] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          uint32_t q[4];
#pragma unroll
          for (int m = 0; m < 4; ++m)
            q[m] = pack_bf16x2(w[2 * m] * bf16_at(xr[k][2 * m], s),
                               w[2 * m + 1] * bf16_at(xr[k][2 * m + 1], s));
          st16(sX + (8 * cb + s) * C::QP + 8 * jb, make_uint4(q[0], q[1], q[2], q[3]));
        }
      }
    }
  };

  const int wn = wave % C::WN, wp = wave / C::WN;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int ksteps = (rows + 31) / 32;

  load_x(h0);
  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    __syncthreads();  // previous head's products are done reading sX
    store_x();
    __syncthreads();
    if (hh + 1 < HB) load_x(h + 1);  // in flight during the products below

    f32x4_t acc[C::TN][C::TP];
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int tp = 0; tp < C::TP; ++tp) acc[tn][tp] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int ks = 0; ks < ksteps; ++ks) {
      const int k0 = ks * 32 + 8 * g4;
      bf16x8_t a[C::TN], bb[C::TP];
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
        a[tn] = as_bf16x8(ld16(sB + ((wn * C::TN + tn) * 16 + r16) * C::QP + k0));
#pragma unroll
      for (int tp = 0; tp < C::TP; ++tp) {
        const int pt = wp * C::TP + tp;
        bb[tp] = pt < C::NT_P ? as_bf16x8(ld16(sX + (pt * 16 + r16) * C::QP + k0))
                              : as_bf16x8(make_uint4(0, 0, 0, 0));
      }
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
        for (int tp = 0; tp < C::TP; ++tp) acc[tn][tp] = mfma_16x16x32(a[tn], bb[tp], acc[tn][tp]);
    }

    // lane holds S^T[n = 4*g4 + i][p = r16] of each tile: four consecutive n
    uint16_t* out = states + ((b * H + h) * nc + c) * (int64_t)P * N;
#pragma unroll
    for (int tp = 0; tp < C::TP; ++tp) {
      const int pt = wp * C::TP + tp;
      if (pt < C::NT_P) {
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
  }
}

// Heads per workgroup: a divisor of the heads in one B/C group, as large as
// keeps the grid at >= 1024 workgroups (4 per compute unit), at most 8.
int pick_heads_per_wg(const Plan& p, int nnb) {
  const int64_t hpg = p.H / p.G;
  const int64_t base = p.batch * p.nc * nnb * p.H;
  int hb = 1;
  while (hb < 8 && hpg % (hb * 2) == 0 && base / (hb * 2) >= 1024) hb *= 2;
  return hb;
}

template <int P, int NB, int Q>
hipError_t launch_pnq(const Plan& p, const void* x, const void* B, const float* cs,
                      const float* dtc, void* st, hipStream_t s) {
  const int nnb = (int)(p.N / NB);
  const int hb = pick_heads_per_wg(p, nnb);
  const int64_t grid = p.batch * p.nc * (p.H / hb) * nnb;
  chunk_state_mfma_kernel<P, NB, Q><<<dim3((unsigned)grid), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), cs, dtc,
      static_cast<uint16_t*>(st), p.L, (int)p.H, (int)p.G, (int)p.N, p.nc, hb);
  return hipGetLastError();
}

template <int P, int NB>
hipError_t launch_pn(const Plan& p, const void* x, const void* B, const float* cs,
                     const float* dtc, void* st, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_pnq<P, NB, 64>(p, x, B, cs, dtc, st, s);
    case 128: return launch_pnq<P, NB, 128>(p, x, B, cs, dtc, st, s);
    case 256: return launch_pnq<P, NB, 256>(p, x, B, cs, dtc, st, s);
    default: return hipErrorInvalidValue;
  }
}

template <int P>
hipError_t launch_p(const Plan& p, const void* x, const void* B, const float* cs,
                    const float* dtc, void* st, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_pn<P, 16>(p, x, B, cs, dtc, st, s);
    case 32: return launch_pn<P, 32>(p, x, B, cs, dtc, st, s);
    case 64: return launch_pn<P, 64>(p, x, B, cs, dtc, st, s);
    default: return launch_pn<P, 128>(p, x, B, cs, dtc, st, s);  // 128, 256
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
  switch (p.P) {
    case 16: return launch_p<16>(p, x, B, dA_cs, dtc, states, s);
    case 32: return launch_p<32>(p, x, B, dA_cs, dtc, states, s);
    case 64: return launch_p<64>(p, x, B, dA_cs, dtc, states, s);
    case 128: return launch_p<128>(p, x, B, dA_cs, dtc, states, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
