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
// Mapping (one workgroup of four wavefronts, one per SIMD, per (b, c) and HB
// heads of one B/C group):
//  * Products are computed transposed, Y^T[p][i], so the score tile never
//    leaves registers: G^T[j][i] = B_j . C_i comes out of the matrix cores
//    with each lane holding one column i and four consecutive rows j, which
//    is the layout of the B operand of the next product Y^T += X^T W^T (two
//    16-row tiles of G^T form one 32-deep operand; x fragments are read from
//    LDS in the same j order).
//  * G^T (the C B^T of the pages' dual form) depends only on the group: it is
//    computed once per workgroup, from B staged through LDS, and reused by
//    the HB heads; only the decay mask is per head. It is held as packed bf16
//    (rounded once more after the decay is applied).
//  * The R = Q/16 row groups of 16 rows are dealt out zigzag: with Q = 256,
//    wavefront w owns row groups w, 7-w, 8+w, 15-w, whose causal tile counts
//    add up to the same 34 for every wavefront. One x fragment read from LDS
//    feeds all of a wavefront's row groups.
//  * The decay exp(l_i - l_j) is never formed from exp(l_i) * exp(-l_j)
//    (that overflows); off-diagonal tiles use a factorisation through the
//    tile boundaries, exp(l_i - l_r0) * exp(l_r0 - l_te) * exp(l_te - l_j),
//    with r0 the first row of the row group and te the last row of the
//    column tile, every factor <= 1; diagonal tiles are masked (j > i -> 0)
//    before the exponential of l_i - l_j is taken.
//  * Per head, x (transposed) and Hin are staged in LDS in fragment-major
//    order: each lane's 16-byte operand fragment is contiguous, so a matrix
//    core operand is one conflict-free 16-byte LDS read; a swizzle of the
//    lane slot inside each 1 KB fragment block spreads the staging writes
//    over the banks. x, Hin, l and dt of the next head are loaded into
//    registers while the current head's products run.
//  * The skip term D_h x_i is added in fp32 in the epilogue.
#include "mfma_common.h"

namespace ssd {
namespace {

template <int P, int N, int Q>
struct ScanCfg {
  static constexpr int R = Q / 16;            // row groups of 16
  static constexpr int NM = Q / 32;           // 32-deep steps over the chunk positions
  static constexpr int RG = 2;                // row groups per wavefront (a zigzag pair)
  static constexpr int WAVES = R / RG;        // 2, 4 or 8
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NTP = P / 16;          // p tiles
  static constexpr int NK = (N + 31) / 32;    // 32-deep steps over n
  static constexpr int NGT = R - 1;           // off-diagonal G^T tiles per wavefront
  static constexpr int XBLK = (Q / 4) * (P / 8);  // 4x8 blocks of the x tile
  static constexpr int XPT = (XBLK + THREADS - 1) / THREADS;
  static constexpr int HCH = P * N / 8;           // 16-byte chunks of Hin
  static constexpr int HPT = (HCH + THREADS - 1) / THREADS;
  static constexpr int FPT = (Q + THREADS - 1) / THREADS;
  static constexpr int NSL = (N + 127) / 128;     // n slices when staging B
  static constexpr int NSW = N < 128 ? N : 128;   // width of one slice
  static constexpr int BPITCH = NSW + 8;          // staged B row pitch (bf16)
  // LDS carve-up (bytes)
  static constexpr int X_BYTES = NTP * NM * 64 * 16;
  static constexpr int H_BYTES = NTP * NK * 64 * 16;
  static constexpr int XN_PITCH = P + 8;          // natural-layout x row pitch (bf16)
  static constexpr int XN_BYTES = Q * XN_PITCH * 2;
  static constexpr int C_BYTES = WAVES * RG * NK * 64 * 16;
  static constexpr int F_BYTES = 3 * Q * 4;
  static constexpr int BST_BYTES = Q * BPITCH * 2;
  // LDS per workgroup such that eight wavefronts (two per SIMD) share a CU
  static constexpr int LIMIT = 160 * 1024 / (8 / WAVES);
  static constexpr bool USE_XN = X_BYTES + H_BYTES + F_BYTES + XN_BYTES <= LIMIT;
  static constexpr int BASE = X_BYTES + H_BYTES + F_BYTES + (USE_XN ? XN_BYTES : 0);
  static constexpr int REST = BASE > BST_BYTES ? BASE : BST_BYTES;
  static constexpr bool PARK_C = C_BYTES + REST <= LIMIT;
  static constexpr int C_SZ = PARK_C ? C_BYTES : 0;
  static constexpr int TOTAL = C_SZ + REST;
  // offsets: [C frags][x frags][Hin frags][l, dt, col][x natural]; the B
  // staging area aliases everything after the C fragments (it is used
  // before any of those buffers)
  static constexpr int OFF_C = 0;
  static constexpr int OFF_X = C_SZ, OFF_H = OFF_X + X_BYTES, OFF_F = OFF_H + H_BYTES;
  static constexpr int OFF_XN = OFF_F + F_BYTES;
  static constexpr int OFF_B = C_SZ;
};

template <int Q>
constexpr int kScanThreads = 2 * Q;  // Q/32 wavefronts of two row groups each

// Slot of lane (r16, g4) inside a 1 KB fragment block. Readers cover all 64
// slots of a block, so any per-block permutation keeps their reads
// conflict-free; these two spread the staging writes across the banks.
__device__ __forceinline__ int xslot(int r16, int g4, int pt) { return 16 * g4 + ((r16 + g4 + 4 * pt) & 15); }
__device__ __forceinline__ int hslot(int r16, int g4) { return 16 * g4 + ((r16 + 4 * g4) & 15); }

template <int P, int N, int Q>
__global__ __launch_bounds__(kScanThreads<Q>) __attribute__((amdgpu_waves_per_eu(2))) void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dA_cs, const float* __restrict__ dtc,
    const uint16_t* __restrict__ states, uint16_t* __restrict__ y,
    int64_t L, int H, int G, int64_t nc, int HB) {
  using C = ScanCfg<P, N, Q>;
  constexpr int R = C::R, NM = C::NM, RG = C::RG, NTP = C::NTP, NK = C::NK;
  __shared__ __align__(16) unsigned char lds[C::TOTAL];
  uint4* sXf = reinterpret_cast<uint4*>(lds + C::OFF_X);   // x^T fragments [pt][m][slot]
  uint4* sHf = reinterpret_cast<uint4*>(lds + C::OFF_H);   // Hin fragments [pt][ks][slot]
  float* sL = reinterpret_cast<float*>(lds + C::OFF_F);    // l_j
  float* sDt = sL + Q;                                     // dt_j
  float* sCol = sL + 2 * Q;                                // exp(l_{16*floor(j/16)+15} - l_j) * dt_j
  uint16_t* sXn = reinterpret_cast<uint16_t*>(lds + C::OFF_XN);  // x [j][p] (when it fits)
  uint4* sCf = reinterpret_cast<uint4*>(lds + C::OFF_C);   // C fragments per wavefront (when parked)
  uint16_t* sB = reinterpret_cast<uint16_t*>(lds + C::OFF_B);  // staged B slice [j][n] (setup only)

  const int nhg = H / HB;
  int64_t bid = xcd_local_order(blockIdx.x, gridDim.x);
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
  const int64_t t0 = c * Q;
  const int rows = (int)(L - t0 < Q ? L - t0 : Q);

  // row groups of this wavefront: w and R-1-w (w + 1 and R - w causal tiles)
  int rk[RG], ik[RG];
  rk[0] = wave;
  rk[1] = R - 1 - wave;
#pragma unroll
  for (int k = 0; k < RG; ++k) ik[k] = 16 * rk[k] + r16;
  // G^T slot of off-diagonal tile t of row group k, static for static k and
  // t: row group 0 fills slots 0.. upwards, row group 1 fills R-2.. downwards
  // (its tile t at slot R-2-t), and the two runs meet without overlap.
  auto gslot = [&](int k, int t) {
    const int sidx = k == 0 ? t : R - 2 - t;
    return sidx < 0 ? 0 : (sidx > C::NGT - 1 ? C::NGT - 1 : sidx);
  };

  // ---- C fragments of the row groups (B operand: column i, 8 consecutive n) ----
  bf16x8_t Cr[RG][NK];
#pragma unroll
  for (int k = 0; k < RG; ++k)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int n = 32 * ks + 8 * g4;
      const bool ok = n < N && ik[k] < rows;
      Cr[k][ks] = as_bf16x8(ld16_keep(Cm + ((b * L + t0 + min(ik[k], rows - 1)) * G + g) * N + (n < N ? n : 0), ok));
    }

  // C fragments parked in this wavefront's LDS region (when they fit): the
  // G^T set-up below and every head's chunk-output product read them there.
  uint4* cpark = sCf + wave * (RG * NK * 64);
  if constexpr (C::PARK_C) {
#pragma unroll
    for (int k = 0; k < RG; ++k)
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) cpark[(k * NK + ks) * 64 + lane] = __builtin_bit_cast(uint4, Cr[k][ks]);
  }

  // ---- G^T = B C^T for every tile a row group needs, B staged through LDS.
  // Slot e < NGT holds an off-diagonal tile; slot NGT + k the diagonal tile of
  // row group k. Which (row group, tile) a slot holds depends on the
  // wavefront only, so the loop over slots is static and branch-free. ----
  auto slot_rg_tile = [&](int e, int& k, int& t) {
    if (e >= C::NGT) {
      k = e - C::NGT;
      t = rk[k];
      return;
    }
    if (e < rk[0]) {
      k = 0;
      t = e;
    } else {
      k = 1;
      t = R - 2 - e;
    }
  };
  f32x4_t Gacc[C::NGT + RG];
#pragma unroll
  for (int e = 0; e < C::NGT + RG; ++e) Gacc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sl = 0; sl < C::NSL; ++sl) {
    __syncthreads();
    constexpr int CH = Q * C::NSW / 8;  // 16-byte chunks of the slice
#pragma unroll
    for (int q = 0; q < (CH + C::THREADS - 1) / C::THREADS; ++q) {
      const int ci = tid + q * C::THREADS;
      if (ci < CH) {
        const int j = ci / (C::NSW / 8), n0 = 8 * (ci % (C::NSW / 8));
        st16(sB + j * C::BPITCH + n0,
             ld16_keep(Bm + ((b * L + t0 + min(j, rows - 1)) * G + g) * N + sl * 128 + n0, j < rows));
      }
    }
    __syncthreads();
    int srow[C::NGT + RG], sk[C::NGT + RG];
#pragma unroll
    for (int e = 0; e < C::NGT + RG; ++e) {
      int k, t;
      slot_rg_tile(e, k, t);
      // slots whose tile a row group does not need (RG == 1 tail) stay unused
      srow[e] = 16 * (t < 0 ? 0 : (t > R - 1 ? R - 1 : t)) + r16;
      sk[e] = k;
    }
#pragma unroll
    for (int kk = 0; kk < C::NSW / 32 + (C::NSW < 32 ? 1 : 0); ++kk) {
      const int ks = sl * 4 + kk;
      const int nl = 32 * kk + 8 * g4;
#pragma unroll
      for (int e = 0; e < C::NGT + RG; ++e) {
        const bf16x8_t bfrag =
            as_bf16x8(nl < C::NSW ? ld16(sB + srow[e] * C::BPITCH + nl) : make_uint4(0, 0, 0, 0));
        bf16x8_t cfrag;
        if constexpr (C::PARK_C) {
          cfrag = as_bf16x8(cpark[(sk[e] * NK + ks) * 64 + lane]);
        } else {
          cfrag = Cr[0][ks];
#pragma unroll
          for (int k2 = 1; k2 < RG; ++k2)
            if (sk[e] == k2) cfrag = Cr[k2][ks];
        }
        Gacc[e] = mfma_16x16x32(bfrag, cfrag, Gacc[e]);
      }
    }
  }
  uint2 Gt[C::NGT], Gd[RG];
#pragma unroll
  for (int e = 0; e < C::NGT; ++e)
    Gt[e] = make_uint2(pack_bf16x2(Gacc[e][0], Gacc[e][1]), pack_bf16x2(Gacc[e][2], Gacc[e][3]));
#pragma unroll
  for (int k = 0; k < RG; ++k)
    Gd[k] = make_uint2(pack_bf16x2(Gacc[C::NGT + k][0], Gacc[C::NGT + k][1]),
                       pack_bf16x2(Gacc[C::NGT + k][2], Gacc[C::NGT + k][3]));
  __syncthreads();  // the B staging area is reused below

  // ---- per-head inputs: global -> registers (one head ahead) -> LDS ----
  uint4 xr[C::XPT][4];
  uint4 hr[C::HPT];
  float lpre[C::FPT], dpre[C::FPT];
  float dnext = 0.f;
  auto fetch_head = [&](int h) {
    dnext = D != nullptr ? D[h] : 0.f;
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * C::THREADS;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          // raw load (clamped row, always in bounds); rows past the end are
          // zeroed when staged, so nothing here waits for the data
          const int j = 4 * jb + rr;
          xr[k][rr] = ld16(x + ((b * L + t0 + min(j, rows - 1)) * H + h) * P + 8 * cb);
        }
      }
    }
    const uint16_t* hin = states + ((b * H + h) * nc + c) * (int64_t)P * N;
#pragma unroll
    for (int k = 0; k < C::HPT; ++k) {
      const int ci = tid + k * C::THREADS;
      if (ci < C::HCH) hr[k] = ld16(hin + 8 * ci);
    }
    const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
    const float* dc = dtc + ((b * H + h) * nc + c) * Q;
#pragma unroll
    for (int k = 0; k < C::FPT; ++k) {
      const int i = tid + k * C::THREADS;
      if (i < Q) {
        lpre[k] = lc[i];
        dpre[k] = dc[i];
      }
    }
  };
  auto stage_head = [&]() {
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = tid + k * C::THREADS;
      if (bi < C::XBLK) {
        const int cb = bi % (P / 8), jb = bi / (P / 8);
        const int j0 = 4 * jb;
        const int m = j0 >> 5, half = (j0 >> 4) & 1, jg = (j0 >> 2) & 3;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (j0 + rr >= rows) xr[k][rr] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 8; ++s) {  // column p = 8cb + s: four bf16 along j
          const uint32_t sel = (s & 1) ? 0x07060302u : 0x05040100u;
          const int mw = s >> 1;
          auto word = [&](const uint4& v) { return mw == 0 ? v.x : mw == 1 ? v.y : mw == 2 ? v.z : v.w; };
          const uint32_t w0 = __builtin_amdgcn_perm(word(xr[k][1]), word(xr[k][0]), sel);
          const uint32_t w1 = __builtin_amdgcn_perm(word(xr[k][3]), word(xr[k][2]), sel);
          const int p = 8 * cb + s;
          const int pt = p >> 4;
          uint4* blk = sXf + (pt * NM + m) * 64;
          reinterpret_cast<uint2*>(blk + xslot(p & 15, jg, pt))[half] = make_uint2(w0, w1);
        }
        if constexpr (C::USE_XN) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) st16(sXn + (j0 + rr) * C::XN_PITCH + 8 * cb, xr[k][rr]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < C::HPT; ++k) {
      const int ci = tid + k * C::THREADS;
      if (ci < C::HCH) {
        const int p = ci / (N / 8), n0 = 8 * (ci % (N / 8));
        sHf[((p >> 4) * NK + (n0 >> 5)) * 64 + hslot(p & 15, (n0 >> 3) & 3)] = hr[k];
      }
    }
#pragma unroll
    for (int k = 0; k < C::FPT; ++k) {
      const int i = tid + k * C::THREADS;
      if (i < Q) {  // Q is a multiple of 64: whole wavefronts take this branch
        const float lend = __shfl(lpre[k], lane | 15, 64);  // l at the end of the 16-row tile
        sL[i] = lpre[k];
        sDt[i] = dpre[k];
        sCol[i] = __expf(lend - lpre[k]) * dpre[k];
      }
    }
  };

  if (N < 32) {  // fragment slots past N stay zero for the whole workgroup
    for (int e = tid; e < NTP * NK * 64; e += C::THREADS) sHf[e] = make_uint4(0, 0, 0, 0);
  }
  // The loop is rotated by hand: head h's inputs are staged at the end of
  // iteration h-1, after its stores, so the only path into each staging step
  // has the same loads and stores outstanding and the wait for the prefetched
  // inputs does not also wait for the y stores that follow them.
  fetch_head(h0);
  stage_head();
  __syncthreads();
  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    const float dh = dnext;
    // in flight during this head's products (the last head re-reads itself,
    // which keeps the memory-operation count the same on every iteration)
    fetch_head(hh + 1 < HB ? h + 1 : h);

    // per-wavefront decay scalars
    float lk[RG], rf[RG], el[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      lk[k] = sL[ik[k]];
      el[k] = __expf(lk[k]);
      rf[k] = __expf(lk[k] - sL[16 * rk[k]]);
    }
    float tv = 0.f;  // lane 16k + t: exp(l_{16 r_k} - l_{16t+15}) for t < r_k
    {
      const int k = lane >> 4, t = lane & 15;
      int rr = -1;
#pragma unroll
      for (int kk = 0; kk < RG; ++kk)
        if (kk == k) rr = rk[kk];
      if (t < rr) tv = __expf(sL[16 * rr] - sL[16 * t + 15]);
    }
    f32x4_t acc[RG][NTP];
    // chunk output: Y^T[p][i] = sum_n Hin[p][n] C_i[n], scaled by exp(l_i)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      bf16x8_t ck[RG];
#pragma unroll
      for (int k = 0; k < RG; ++k) ck[k] = C::PARK_C ? as_bf16x8(cpark[(k * NK + ks) * 64 + lane]) : Cr[k][ks];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) {
        const bf16x8_t a = as_bf16x8(sHf[(pt * NK + ks) * 64 + hslot(r16, g4)]);
#pragma unroll
        for (int k = 0; k < RG; ++k)
          acc[k][pt] = mfma_16x16x32(a, ck[k], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[k][pt]);
      }
    }
#pragma unroll
    for (int k = 0; k < RG; ++k)
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] *= el[k];

    // intra-chunk, off-diagonal tiles: all row groups walk the same pairs of
    // column tiles (2kp, 2kp+1), so one x fragment feeds every row group.
    // All factors are <= 1: exp(l_i - l_r0) * exp(l_r0 - l_te) * c_j.
    auto xfrag = [&](int m, int pt) { return sXf[(pt * NM + m) * 64 + xslot(r16, g4, pt)]; };
    auto colf = [&](int t) { return *reinterpret_cast<const float4*>(sCol + 16 * t + 4 * g4); };
    auto wpair = [&](uint2 ga, float sa, float4 ca, uint2 gb, float sb, float4 cb) {
      const float w0 = bf16_lo(ga.x) * sa * ca.x, w1 = bf16_hi(ga.x) * sa * ca.y;
      const float w2 = bf16_lo(ga.y) * sa * ca.z, w3 = bf16_hi(ga.y) * sa * ca.w;
      const float w4 = bf16_lo(gb.x) * sb * cb.x, w5 = bf16_hi(gb.x) * sb * cb.y;
      const float w6 = bf16_lo(gb.y) * sb * cb.z, w7 = bf16_hi(gb.y) * sb * cb.w;
      return as_bf16x8(make_uint4(pack_bf16x2(w0, w1), pack_bf16x2(w2, w3), pack_bf16x2(w4, w5),
                                  pack_bf16x2(w6, w7)));
    };
    auto lanef = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tv), l)); };

#pragma unroll
    for (int kp = 0; kp < NM; ++kp) {
      const int ta = 2 * kp, tb = 2 * kp + 1;
      if (ta >= rk[1]) break;  // wavefront-uniform: row group 1 has the most tiles
      uint4 a[NTP];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) a[pt] = xfrag(kp, pt);
      const float4 ca = colf(ta), cb = colf(tb);
#pragma unroll
      for (int k = 0; k < RG; ++k) {
        if (ta < rk[k]) {  // tile tb == r_k is the diagonal: excluded here
          const float sa = rf[k] * lanef(16 * k + ta);
          const float sb = tb < rk[k] ? rf[k] * lanef(16 * k + tb) : 0.f;
          const bf16x8_t w = wpair(Gt[gslot(k, ta)], sa, ca, Gt[gslot(k, tb)], sb, cb);
#pragma unroll
          for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(as_bf16x8(a[pt]), w, acc[k][pt]);
        }
      }
    }

    // diagonal tiles: mask (j > i) before the exponential
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const int t = rk[k], i = ik[k];
      const int j0 = 16 * t + 4 * g4;
      const float4 lj = *reinterpret_cast<const float4*>(sL + j0);
      const float4 dj = *reinterpret_cast<const float4*>(sDt + j0);
      const float ljv[4] = {lj.x, lj.y, lj.z, lj.w};
      const float djv[4] = {dj.x, dj.y, dj.z, dj.w};
      const uint2 gp = Gd[k];
      const float gv[4] = {bf16_lo(gp.x), bf16_hi(gp.x), bf16_lo(gp.y), bf16_hi(gp.y)};
      float w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jq = j0 + q;
        const float e = __expf(jq <= i ? lk[k] - ljv[q] : -INFINITY);
        w[q] = gv[q] * e * djv[q];
      }
      const uint32_t w01 = pack_bf16x2(w[0], w[1]), w23 = pack_bf16x2(w[2], w[3]);
      const bool upper = t & 1;  // which half of the 32-deep pair holds tile t
      const bf16x8_t wop = as_bf16x8(upper ? make_uint4(0, 0, w01, w23) : make_uint4(w01, w23, 0, 0));
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(as_bf16x8(xfrag(t >> 1, pt)), wop, acc[k][pt]);
    }

    // epilogue: + D_h x_i in fp32, store; lane holds Y^T[p = 16pt + 4g4 + q][i].
    // Rows past the end of the sequence fall outside the buffer range and are
    // dropped, so the store sequence is the same for every chunk.
    uint16_t* ybase = y + ((b * L + t0) * H + h) * P;
    const __amdgpu_buffer_rsrc_t yr = buffer_range(ybase, (uint32_t)(((rows - 1) * (int64_t)H + 1) * P * 2));
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const int i = ik[k];
      const uint32_t rowoff = (uint32_t)(i * (int64_t)H * P * 2);
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) {
        const int p = 16 * pt + 4 * g4;
        float xv[4];
        if constexpr (C::USE_XN) {
          const uint2 xx = *reinterpret_cast<const uint2*>(sXn + i * C::XN_PITCH + p);
          xv[0] = bf16_lo(xx.x); xv[1] = bf16_hi(xx.x); xv[2] = bf16_lo(xx.y); xv[3] = bf16_hi(xx.y);
        } else {
          const unsigned char* xb = reinterpret_cast<const unsigned char*>(sXf);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int pq = p + q;
            const int o = (((pq >> 4) * NM + (i >> 5)) * 64 + xslot(pq & 15, (i >> 2) & 3, pq >> 4)) * 16 +
                          ((i >> 4) & 1) * 8 + (i & 3) * 2;
            xv[q] = __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t*>(xb + o)) << 16);
          }
        }
        const f32x4_t v = acc[k][pt];
        const float o0 = fmaf(dh, xv[0], v[0]), o1 = fmaf(dh, xv[1], v[1]);
        const float o2 = fmaf(dh, xv[2], v[2]), o3 = fmaf(dh, xv[3], v[3]);
        buffer_st8(make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)), yr, rowoff + p * 2);
      }
    }
    __syncthreads();  // every wavefront is done with this head's LDS tiles
    if (hh + 1 < HB) {
      stage_head();
      __syncthreads();
    }
  }
}

// Heads per workgroup: a divisor of the heads in one B/C group, at most 8,
// as large as keeps at least two workgroups per compute unit (the G^T set-up
// is amortised over more heads; one workgroup fills a compute unit's LDS).
int pick_heads_per_wg(const Plan& p) {
  const int64_t hpg = p.H / p.G;
  const int64_t base = p.batch * p.nc * p.H;
  int hb = 1;
  while (hb < 8 && hpg % (hb * 2) == 0 && base / (hb * 2) >= 512) hb *= 2;
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
  // byte offsets inside one chunk's rows of y must fit the 32-bit buffer range
  if (int64_t(p.Q) * p.H * p.P * 2 >= (int64_t(1) << 31)) return false;
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
