// Steps 4+5 on bf16 matrix cores: the output of every chunk.
//
// Inside a chunk the semiseparable matrix is contracted in its dense, masked
// (attention-like) order, and the state entering the chunk adds its
// contribution ("Mamba-2 vs Transformers: SSMs, structured state space
// duality", sections "How we compared ..." and "Mamba-2 and the SSD paper:
// what changed in practice", contraction-order table). For row i of chunk c:
//     y_i = sum_{j<=i} exp(l_i - l_j) dt_j (C_i . B_j) x_j      (intra-chunk)
//         + exp(l_i) Hin_c C_i                                   (chunk output)
//         + D_h x_i
//
// Mapping (per workgroup: one (b, c) and HB heads of one B/C group):
//  * Products are computed transposed, Y^T[p][i], so the score tile can stay
//    in registers: G^T[j][i] = B_j . C_i is produced by the matrix cores with
//    each lane holding one column i and four consecutive rows j, which is
//    exactly the layout of the B operand of the next product Y^T += X^T W^T
//    (two 16-row tiles of G^T make one 32-deep operand; the x fragments are
//    read from LDS in the same j order).
//  * G^T (the C B^T of the pages' dual form) depends only on the group, so it
//    is computed once per workgroup and reused by its HB heads; only the
//    decay mask is per head.
//  * The chunk's rows are cut into R = Q/16 row groups of 16. Wavefront w
//    owns row groups r1 = 2w+1 and r2 = R-2-2w: an odd/even pair whose causal
//    tile counts add up to R+1, so every wavefront does the same work, and
//    both counts stay even-aligned so tiles pair into 32-deep operands.
//  * The decay exp(l_i - l_j) is never formed from exp(l_i) * exp(-l_j)
//    (that overflows); off-diagonal tiles use a factorisation through the
//    tile boundaries, exp(l_i - l_r0) * exp(l_r0 - l_te) * exp(l_te - l_j),
//    with r0 the first row of the row group and te the last row of the
//    column tile, every factor <= 1; diagonal tiles are masked (j > i -> 0)
//    before the exponential of l_i - l_j is taken.
//  * x of each head is staged in LDS transposed ([p][j]); Hin ([p][n]) in
//    its natural layout; both are prefetched into registers for the next
//    head while the current head's products run.
#include "mfma_common.h"

namespace ssd {
namespace {

template <int P, int N, int Q>
struct ScanCfg {
  static constexpr int R = Q / 16;          // row groups of 16
  static constexpr int WAVES = R / 2;       // two row groups per wavefront
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NTP = P / 16;        // p tiles
  static constexpr int NK = (N + 31) / 32;  // 32-deep steps over n
  static constexpr int QP = Q + 8;          // LDS pitch of x^T rows (bf16)
  static constexpr int NP = NK * 32 + 8;    // LDS pitch of Hin rows (bf16)
  static constexpr int XBLK = (Q / 4) * (P / 8);  // 4x8 blocks of the x tile
  static constexpr int XPT = (XBLK + THREADS - 1) / THREADS;
  static constexpr int HCH = P * N / 8;           // 16-byte chunks of Hin
  static constexpr int HPT = (HCH + THREADS - 1) / THREADS;
};

// workgroup size: two 16-row groups per wavefront
template <int Q>
constexpr int kScanThreads = Q / 32 * 64;

template <int P, int N, int Q>
__global__ __launch_bounds__(kScanThreads<Q>) void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dA_cs, const float* __restrict__ dtc,
    const uint16_t* __restrict__ states, uint16_t* __restrict__ y,
    int64_t L, int H, int G, int64_t nc, int HB) {
  using C = ScanCfg<P, N, Q>;
  constexpr int R = C::R;
  __shared__ __align__(16) uint16_t sX[P * C::QP];
  __shared__ __align__(16) uint16_t sH[P * C::NP];
  __shared__ __align__(16) float sL[Q];     // l_i
  __shared__ __align__(16) float sDt[Q];    // dt_j
  __shared__ __align__(16) float sEl[Q];    // exp(l_i)
  __shared__ __align__(16) float sRow[Q];   // exp(l_i - l_{16*floor(i/16)})
  __shared__ __align__(16) float sCol[Q];   // exp(l_{16*floor(j/16)+15} - l_j) * dt_j
  __shared__ float sT[R * R];               // exp(l_{16r} - l_{16t+15}), t < r

  const int nhg = H / HB;
  int64_t bid = blockIdx.x;
  const int hg = (int)(bid % nhg);
  bid /= nhg;
  const int64_t c = bid % nc;
  const int64_t b = bid / nc;
  const int h0 = hg * HB;
  const int g = h0 / (H / G);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int64_t t0 = c * Q;
  const int rows = (int)(L - t0 < Q ? L - t0 : Q);

  const int r1 = 2 * wave + 1;
  const int r2 = R - 2 - 2 * wave;
  const int i1 = 16 * r1 + r16, i2 = 16 * r2 + r16;

  // ---- C fragments of both row groups (B operand: column i, 8 consecutive n) ----
  bf16x8_t C1[C::NK], C2[C::NK];
#pragma unroll
  for (int ks = 0; ks < C::NK; ++ks) {
    const int n = 32 * ks + 8 * g4;
    const bool nok = n < N;
    C1[ks] = as_bf16x8(nok && i1 < rows ? ld16(Cm + ((b * L + t0 + i1) * G + g) * N + n) : make_uint4(0, 0, 0, 0));
    C2[ks] = as_bf16x8(nok && i2 < rows ? ld16(Cm + ((b * L + t0 + i2) * G + g) * N + n) : make_uint4(0, 0, 0, 0));
  }

  // ---- G^T tiles: k = 0..r1 -> (row group r1, column tile k); k = r1+1..R -> (r2, k-r1-1) ----
  f32x4_t Gt[R + 1];
#pragma unroll
  for (int k = 0; k <= R; ++k) {
    const bool in2 = k > r1;
    const int t = in2 ? k - r1 - 1 : k;
    const int j = 16 * t + r16;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::NK; ++ks) {
      const int n = 32 * ks + 8 * g4;
      const bf16x8_t bfrag = as_bf16x8(n < N && j < rows ? ld16(Bm + ((b * L + t0 + j) * G + g) * N + n)
                                                          : make_uint4(0, 0, 0, 0));
      acc = mfma_16x16x32(bfrag, in2 ? C2[ks] : C1[ks], acc);
    }
    Gt[k] = acc;
  }

  // ---- per-head staging: global -> registers (prefetch) -> LDS ----
  uint4 hr[C::HPT];
  uint4 xfull[C::XPT][4];
  auto fetch_head = [&](int h) {
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * C::THREADS;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int j = 4 * jb + rr;
          xfull[k][rr] = j < rows ? ld16(x + ((b * L + t0 + j) * H + h) * P + 8 * cb) : make_uint4(0, 0, 0, 0);
        }
      }
    }
    const uint16_t* hin = states + ((b * H + h) * nc + c) * (int64_t)P * N;
#pragma unroll
    for (int k = 0; k < C::HPT; ++k) {
      const int ci = tid + k * C::THREADS;
      if (ci < C::HCH) hr[k] = ld16(hin + 8 * ci);
    }
  };
  auto stage_head = [&]() {
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * C::THREADS;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
        // column s of the 4x8 block -> 4 bf16 along j
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t sel = (s & 1) ? 0x07060302u : 0x05040100u;
          const int m = s >> 1;
          auto word = [&](const uint4& v) { return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w; };
          const uint32_t w0 = __builtin_amdgcn_perm(word(xfull[k][1]), word(xfull[k][0]), sel);
          const uint32_t w1 = __builtin_amdgcn_perm(word(xfull[k][3]), word(xfull[k][2]), sel);
          *reinterpret_cast<uint2*>(sX + (8 * cb + s) * C::QP + 4 * jb) = make_uint2(w0, w1);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < C::HPT; ++k) {
      const int ci = tid + k * C::THREADS;
      if (ci < C::HCH) {
        const int p = (8 * ci) / N, n = (8 * ci) % N;
        st16(sH + p * C::NP + n, hr[k]);
      }
    }
  };
  auto stage_factors = [&](int h) {
    const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
    const float* dc = dtc + ((b * H + h) * nc + c) * Q;
    for (int i = tid; i < Q; i += C::THREADS) {
      const float li = lc[i];
      const float dj = dc[i];
      sL[i] = li;
      sDt[i] = dj;
      sEl[i] = __expf(li);
      sRow[i] = __expf(li - lc[i & ~15]);
      sCol[i] = __expf(lc[i | 15] - li) * dj;
    }
    for (int e = tid; e < R * R; e += C::THREADS) {
      const int r = e / R, t = e % R;
      sT[e] = t < r ? __expf(lc[16 * r] - lc[16 * t + 15]) : 0.f;
    }
  };

  fetch_head(h0);
  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    __syncthreads();  // the previous head is done with LDS
    stage_head();
    stage_factors(h);
    __syncthreads();
    if (hh + 1 < HB) fetch_head(h + 1);  // in flight during this head's products

    f32x4_t acc1[C::NTP], acc2[C::NTP];
#pragma unroll
    for (int pt = 0; pt < C::NTP; ++pt) {
      acc1[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc2[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // chunk output: Y^T[p][i] = sum_n Hin[p][n] C_i[n], scaled by exp(l_i) below
#pragma unroll
    for (int ks = 0; ks < C::NK; ++ks) {
      const int n = 32 * ks + 8 * g4;
#pragma unroll
      for (int pt = 0; pt < C::NTP; ++pt) {
        const bf16x8_t a = as_bf16x8(n < N ? ld16(sH + (16 * pt + r16) * C::NP + n) : make_uint4(0, 0, 0, 0));
        acc1[pt] = mfma_16x16x32(a, C1[ks], acc1[pt]);
        acc2[pt] = mfma_16x16x32(a, C2[ks], acc2[pt]);
      }
    }
    const float el1 = sEl[i1], el2 = sEl[i2];
    const float li1 = sL[i1], li2 = sL[i2];
    const float rf1 = sRow[i1], rf2 = sRow[i2];
#pragma unroll
    for (int pt = 0; pt < C::NTP; ++pt) {
      acc1[pt] *= el1;
      acc2[pt] *= el2;
    }

    // intra-chunk: pairs of 16-row column tiles -> one 32-deep operand
#pragma unroll
    for (int kp = 0; kp < (R + 2) / 2; ++kp) {
      const int k = 2 * kp;
      const bool in2 = k > r1;
      const int r = in2 ? r2 : r1;
      const int t = in2 ? k - r1 - 1 : k;
      const int i = in2 ? i2 : i1;
      const float li = in2 ? li2 : li1;
      const float rf = in2 ? rf2 : rf1;
      uint32_t wq[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tt = t + half;
        const f32x4_t gv = (k + half <= R) ? Gt[k + half < R + 1 ? k + half : R] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int j0 = 16 * tt + 4 * g4;
        float w[4];
        if (tt < r) {
          const float s = rf * sT[r * R + tt];
          const float4 cf = *reinterpret_cast<const float4*>(sCol + j0);
          w[0] = gv[0] * s * cf.x;
          w[1] = gv[1] * s * cf.y;
          w[2] = gv[2] * s * cf.z;
          w[3] = gv[3] * s * cf.w;
        } else if (tt == r) {
          const float4 lj = *reinterpret_cast<const float4*>(sL + j0);
          const float4 dj = *reinterpret_cast<const float4*>(sDt + j0);
          const float ljv[4] = {lj.x, lj.y, lj.z, lj.w};
          const float djv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = (j0 + q <= i) ? gv[q] * __expf(li - ljv[q]) * djv[q] : 0.f;
        } else {
          w[0] = w[1] = w[2] = w[3] = 0.f;
        }
        wq[2 * half] = pack_bf16x2(w[0], w[1]);
        wq[2 * half + 1] = pack_bf16x2(w[2], w[3]);
      }
      const bf16x8_t wop = as_bf16x8(make_uint4(wq[0], wq[1], wq[2], wq[3]));
      const int ja = 16 * t + 4 * g4, jb2 = 16 * (t + 1) + 4 * g4;
#pragma unroll
      for (int pt = 0; pt < C::NTP; ++pt) {
        const uint16_t* row = sX + (16 * pt + r16) * C::QP;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + ja);
        const uint2 hi = (t + 1) * 16 < Q ? *reinterpret_cast<const uint2*>(row + jb2) : make_uint2(0, 0);
        const bf16x8_t a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        if (in2)
          acc2[pt] = mfma_16x16x32(a, wop, acc2[pt]);
        else
          acc1[pt] = mfma_16x16x32(a, wop, acc1[pt]);
      }
    }

    // epilogue: + D x, store; lane holds Y^T[p = 16pt + 4g4 + q][i]
    const float dh = D != nullptr ? D[h] : 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int i = half ? i2 : i1;
      if (i < rows) {
        const int64_t off = ((b * L + t0 + i) * H + h) * P;
#pragma unroll
        for (int pt = 0; pt < C::NTP; ++pt) {
          const int p = 16 * pt + 4 * g4;
          const uint2 xv = *reinterpret_cast<const uint2*>(x + off + p);
          const f32x4_t v = half ? acc2[pt] : acc1[pt];
          const float o0 = v[0] + dh * bf16_lo(xv.x);
          const float o1 = v[1] + dh * bf16_hi(xv.x);
          const float o2 = v[2] + dh * bf16_lo(xv.y);
          const float o3 = v[3] + dh * bf16_hi(xv.y);
          *reinterpret_cast<uint2*>(y + off + p) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
      }
    }
  }
}

// Heads per workgroup: a divisor of the heads in one B/C group, as large as
// keeps the grid at >= 1024 workgroups, at most 8.
int pick_heads_per_wg(const Plan& p) {
  const int64_t hpg = p.H / p.G;
  const int64_t base = p.batch * p.nc * p.H;
  int hb = 1;
  while (hb < 8 && hpg % (hb * 2) == 0 && base / (hb * 2) >= 1024) hb *= 2;
  return hb;
}

template <int P, int N, int Q>
hipError_t launch_pnq(const Plan& p, const void* x, const void* B, const void* Cm, const float* D,
                      const float* cs, const float* dtc, const void* st, void* y, hipStream_t s) {
  using Cfg = ScanCfg<P, N, Q>;
  const int hb = pick_heads_per_wg(p);
  const int64_t grid = p.batch * p.nc * (p.H / hb);
  chunk_scan_mfma_kernel<P, N, Q><<<dim3((unsigned)grid), Cfg::THREADS, 0, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(Cm), D,
      cs, dtc, static_cast<const uint16_t*>(st), static_cast<uint16_t*>(y), p.L, (int)p.H, (int)p.G, p.nc, hb);
  return hipGetLastError();
}

template <int P, int N>
hipError_t launch_pn(const Plan& p, const void* x, const void* B, const void* Cm, const float* D,
                     const float* cs, const float* dtc, const void* st, void* y, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_pnq<P, N, 64>(p, x, B, Cm, D, cs, dtc, st, y, s);
    case 128: return launch_pnq<P, N, 128>(p, x, B, Cm, D, cs, dtc, st, y, s);
    case 256: return launch_pnq<P, N, 256>(p, x, B, Cm, D, cs, dtc, st, y, s);
    default: return hipErrorInvalidValue;
  }
}

template <int P>
hipError_t launch_p(const Plan& p, const void* x, const void* B, const void* Cm, const float* D,
                    const float* cs, const float* dtc, const void* st, void* y, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_pn<P, 16>(p, x, B, Cm, D, cs, dtc, st, y, s);
    case 32: return launch_pn<P, 32>(p, x, B, Cm, D, cs, dtc, st, y, s);
    case 64: return launch_pn<P, 64>(p, x, B, Cm, D, cs, dtc, st, y, s);
    case 128: return launch_pn<P, 128>(p, x, B, Cm, D, cs, dtc, st, y, s);
    case 256: return launch_pn<P, 256>(p, x, B, Cm, D, cs, dtc, st, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_chunk_scan_supported(const Plan& p) {
  return p.io == kBF16 && (p.P == 16 || p.P == 32 || p.P == 64 || p.P == 128) &&
         (p.N == 16 || p.N == 32 || p.N == 64 || p.N == 128 || p.N == 256) &&
         (p.Q == 64 || p.Q == 128 || p.Q == 256);
}

hipError_t launch_chunk_scan_mfma(const Plan& p, const void* x, const void* B, const void* Cm,
                                  const float* D, const float* dA_cs, const float* dtc,
                                  const void* states, void* y, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_p<16>(p, x, B, Cm, D, dA_cs, dtc, states, y, s);
    case 32: return launch_p<32>(p, x, B, Cm, D, dA_cs, dtc, states, y, s);
    case 64: return launch_p<64>(p, x, B, Cm, D, dA_cs, dtc, states, y, s);
    case 128: return launch_p<128>(p, x, B, Cm, D, dA_cs, dtc, states, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
