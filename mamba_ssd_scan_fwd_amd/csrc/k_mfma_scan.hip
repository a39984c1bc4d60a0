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
// Mapping: one workgroup per (b, c) and HB heads of one B/C group, with Q/32
// wavefronts (eight at Q = 256: two per SIMD).
//  * Products are computed transposed, Y^T[p][i], so the score tile never
//    leaves registers: G^T[j][i] = B_j . C_i comes out of the matrix cores
//    with each lane holding one column i and four consecutive rows j, which
//    is the layout of the B operand of the next product Y^T += X^T W^T (two
//    16-row tiles of G^T form one 32-deep operand; x fragments are read from
//    LDS in the same j order).
//  * G^T (the C B^T of the pages' dual form) depends only on the group: it is
//    computed once per workgroup and reused by the HB heads, held as packed
//    bf16 in registers; only the decay mask is per head. The C fragments,
//    which also feed the chunk-output product of every head, stay in
//    registers too.
//  * The R = Q/16 row groups of 16 rows are dealt out in pairs: wavefront w
//    owns row groups w and R-1-w, w + 1 and R - w causal tiles, R + 1 for
//    every wavefront.
//  * The decay exp(l_i - l_j) is never formed from exp(l_i) * exp(-l_j)
//    (that overflows). Off-diagonal tiles use a factorisation through the
//    tile boundaries, exp(l_i - l_r0) * exp(l_r0 - l_te) * exp(l_te - l_j),
//    r0 the first row of the row group and te the last row of the column
//    tile, every factor <= 1; the three factors are tabulated per head when
//    its inputs are staged. Diagonal tiles are masked (j > i -> 0) before the
//    exponential of l_i - l_j is taken.
//  * Per head, x (transposed), Hin and the decay tables are staged in LDS,
//    double-buffered: the inputs of head h+1 are loaded into registers while
//    the products of head h run (from one buffer) and are then written to
//    the other buffer. One barrier per head. Operand tiles are fragment-major: each lane's 16-byte operand
//    fragment is contiguous, so a matrix-core operand is one conflict-free
//    16-byte LDS read; a swizzle of the lane slot inside each 1 KB fragment
//    block spreads the staging writes over the banks.
//  * The skip term D_h x_i is one more product on the diagonal tiles' x
//    operand, against D_h times the identity (D_h split into two bf16 parts,
//    so the term is exact to 16 bits of D_h in the fp32 accumulator).
#include "mfma_common.h"

namespace ssd {
namespace {

template <int P, int N, int Q>
struct ScanCfg {
  static constexpr int R = Q / 16;            // row groups of 16
  static constexpr int NM = Q / 32;           // 32-deep steps over the chunk positions
  static constexpr int RG = 2;                // row groups per wavefront
  static constexpr int WAVES = R / RG;        // 2, 4 or 8
  static constexpr int THREADS = WAVES * 64;  // = 2 Q
  static constexpr int NTP = P / 16;          // p tiles
  static constexpr int NK = (N + 31) / 32;    // 32-deep steps over n
  static constexpr int NGT = R - 1;           // off-diagonal G^T tiles per wavefront
  static constexpr int XBLK = (Q / 4) * (P / 8);  // 4x8 blocks of the x tile
  static constexpr int XPT = (XBLK + THREADS - 1) / THREADS;
  static constexpr int HCH = P * N / 8;           // 16-byte chunks of Hin
  static constexpr int HPT = (HCH + THREADS - 1) / THREADS;
  static constexpr int NSL = (N + 127) / 128;     // n slices when staging B
  static constexpr int NSW = N < 128 ? N : 128;   // width of one slice
  static constexpr int BPITCH = NSW + 8;          // staged B row pitch (bf16)
  // one staging buffer (bytes): x^T fragments, Hin fragments, then per
  // position l, dt, (row factor, exp(l)), column factor, and the R x R
  // table of tile-boundary factors
  static constexpr int X_BYTES = NTP * NM * 64 * 16;
  static constexpr int H_BYTES = NTP * NK * 64 * 16;
  static constexpr int OFF_X = 0, OFF_H = X_BYTES, OFF_L = OFF_H + H_BYTES;
  static constexpr int OFF_DT = OFF_L + Q * 4, OFF_RE = OFF_DT + Q * 4;
  static constexpr int OFF_COL = OFF_RE + Q * 8, OFF_T = OFF_COL + Q * 4;
  static constexpr int BUF = OFF_T + R * R * 4;
  static constexpr int BST_BYTES = Q * BPITCH * 2;
  // two buffers when they fit the LDS, else one (and a second barrier per head)
  static constexpr bool DB = 2 * BUF <= 160 * 1024;
  static constexpr int NBUF = DB ? 2 : 1;
  static constexpr int TOTAL = NBUF * BUF > BST_BYTES ? NBUF * BUF : BST_BYTES;
};

template <int Q>
constexpr int kScanThreads = 2 * Q;

// Slot of lane (r16, g4) inside a 1 KB fragment block: a permutation of the
// 64 slots for every block, so the matrix-core operand reads stay
// conflict-free (each group of eight lanes covers the eight 16-byte bank
// positions); the permutations are chosen so that the staging writes of
// eight consecutive lanes land on eight different bank positions too.
//  x^T: eight consecutive staging lanes hold columns p = 8 * cb + s of four
//  p tiles (cb = 0..7): bit 3 of r16 and the p tile pick the position.
__device__ __forceinline__ int xslot(int r16, int g4, int pt) {
  return 16 * g4 + ((r16 & 8) | ((r16 & 7) ^ ((((r16 >> 3) << 2) ^ pt) & 7)));
}
//  Hin: eight consecutive staging lanes hold the four 8-wide n groups of two
//  consecutive 32-deep steps ks of one row p.
__device__ __forceinline__ int hslot(int r16, int g4, int ks) { return 16 * g4 + ((r16 + 2 * g4 + (ks & 1)) & 15); }

template <int P, int N, int Q>
__global__ __launch_bounds__(kScanThreads<Q>) __attribute__((amdgpu_waves_per_eu(2))) void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dA_cs, const float* __restrict__ dtc,
    const uint16_t* __restrict__ states, uint16_t* __restrict__ y,
    int64_t L, int H, int G, int64_t nc, int HB, const ChunkInfo* __restrict__ ctab) {
  using C = ScanCfg<P, N, Q>;
  constexpr int R = C::R, NM = C::NM, RG = C::RG, NTP = C::NTP, NK = C::NK;
  __shared__ __align__(16) unsigned char lds[C::TOTAL];

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
  int64_t row0;  // first token row of this chunk in the [batch * L] arrays
  int rows;      // valid positions in this chunk
  chunk_span(ctab, b, c, L, Q, row0, rows);
  if (rows <= 0) return;  // unused slot of a packed-sequence table (uniform)

  // row groups of this wavefront: w and R-1-w
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

  // ---- C fragments of the row groups (B operand: column i, 8 consecutive n),
  // kept in registers: they also feed the chunk-output product of every head.
  // Rows past the end re-read the last row (their outputs are never stored).
  bf16x8_t Cr[RG][NK];
  {
    const uint16_t* cbase = Cm + (row0 * G + g) * N;
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const uint32_t coff = (uint32_t)((min(ik[k], rows - 1) * G * N + (8 * g4 < N ? 8 * g4 : 0)) * 2);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const uint4 v = ld16_at(cbase, coff + (32 * ks < N ? 64 * ks : 0));
        Cr[k][ks] = as_bf16x8(32 * ks + 8 * g4 < N ? v : make_uint4(0, 0, 0, 0));
      }
    }
  }

  // ---- G^T = B C^T for every tile a row group needs, B staged through LDS.
  // Slot e < NGT holds an off-diagonal tile, slot NGT + k the diagonal tile
  // of row group k; the loop over slots is static and branch-free. ----
  uint16_t* sB = reinterpret_cast<uint16_t*>(lds);
  f32x4_t Gacc[C::NGT + RG];
#pragma unroll
  for (int e = 0; e < C::NGT + RG; ++e) Gacc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int srow[C::NGT + RG], sk[C::NGT + RG];
#pragma unroll
  for (int e = 0; e < C::NGT + RG; ++e) {
    int k, t;
    if (e >= C::NGT) {
      k = e - C::NGT;
      t = rk[k];
    } else if (e < rk[0]) {
      k = 0;
      t = e;
    } else {
      k = 1;
      t = R - 2 - e;
    }
    srow[e] = 16 * t + r16;
    sk[e] = k;
  }
#pragma unroll
  for (int sl = 0; sl < C::NSL; ++sl) {
    if (sl > 0) __syncthreads();
    constexpr int CH = Q * C::NSW / 8;  // 16-byte chunks of the slice
#pragma unroll
    for (int q = 0; q < (CH + C::THREADS - 1) / C::THREADS; ++q) {
      const int ci = tid + q * C::THREADS;
      if (ci < CH) {
        const int j = ci / (C::NSW / 8), n0 = 8 * (ci % (C::NSW / 8));
        st16(sB + j * C::BPITCH + n0,
             ld16_keep(Bm + ((row0 + min(j, rows - 1)) * G + g) * N + sl * 128 + n0, j < rows));
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < C::NSW / 32 + (C::NSW < 32 ? 1 : 0); ++kk) {
      const int ks = sl * 4 + kk;
      const int nl = 32 * kk + 8 * g4;
#pragma unroll
      for (int e = 0; e < C::NGT + RG; ++e) {
        const bf16x8_t bfrag =
            as_bf16x8(nl < C::NSW ? ld16(sB + srow[e] * C::BPITCH + nl) : make_uint4(0, 0, 0, 0));
        const bf16x8_t cfrag = sk[e] == 0 ? Cr[0][ks] : Cr[1][ks];
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
  __syncthreads();  // the B staging area becomes the two head buffers

  // ---- per-head inputs: global -> registers (two heads ahead) -> LDS ----
  uint4 xr[C::XPT][4];
  uint4 hr[C::HPT];
  float lpre = 0.f, dpre = 0.f, tl1 = 0.f, tl2 = 0.f;
  // thread e < R*R tabulates exp(l_{16 r} - l_{16 t + 15}), r = e / R, t = e % R.
  // Staging and fetching use an opaque copy of the thread index, so their
  // per-thread addresses are not kept live through the products.
  // Every load is issued unconditionally, from a clamped (always valid)
  // index where a thread has nothing to fetch: a fixed count of memory
  // operations lets each wait cover exactly the loads it needs.
  auto fetch_head = [&](int h) {
    const int tid = opaque(threadIdx.x);
    const uint16_t* xh = x + (row0 * H + h) * P;
#pragma unroll
    for (int k = 0; k < C::XPT; ++k) {
      const int bi = min(tid + k * C::THREADS, C::XBLK - 1);
      const int cb = bi % (P / 8), jb = bi / (P / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        // raw load (clamped row, always in bounds); rows past the end are
        // zeroed when staged, so nothing here waits for the data
        const int j = 4 * jb + rr;
        xr[k][rr] = ld16_at(xh, (uint32_t)((min(j, rows - 1) * H * P + 8 * cb) * 2));
      }
    }
    const uint16_t* hin = states + ((b * H + h) * nc + c) * (int64_t)P * N;
#pragma unroll
    for (int k = 0; k < C::HPT; ++k) hr[k] = ld16_at(hin, (uint32_t)(16 * min(tid + k * C::THREADS, C::HCH - 1)));
    const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
    const float* dc = dtc + ((b * H + h) * nc + c) * Q;
    const int tq = min(tid, Q - 1), te = min(tid, R * R - 1);
    lpre = ld4f_at(lc, 4 * tq);
    dpre = ld4f_at(dc, 4 * tq);
    tl1 = ld4f_at(lc, 64 * (te / R));
    tl2 = ld4f_at(lc, 64 * (te % R) + 60);
  };
  auto stage_head = [&](unsigned char* buf) {
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63;
    const int tr = tid / R, tt = tid % R;
    uint4* sXf = reinterpret_cast<uint4*>(buf + C::OFF_X);
    uint4* sHf = reinterpret_cast<uint4*>(buf + C::OFF_H);
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
      }
    }
#pragma unroll
    for (int k = 0; k < C::HPT; ++k) {
      const int ci = tid + k * C::THREADS;
      if (ci < C::HCH) {
        const int p = ci / (N / 8), n0 = 8 * (ci % (N / 8));
        sHf[((p >> 4) * NK + (n0 >> 5)) * 64 + hslot(p & 15, (n0 >> 3) & 3, n0 >> 5)] = hr[k];
      }
    }
    float* sL = reinterpret_cast<float*>(buf + C::OFF_L);
    float* sDt = reinterpret_cast<float*>(buf + C::OFF_DT);
    float2* sRE = reinterpret_cast<float2*>(buf + C::OFF_RE);
    float* sCol = reinterpret_cast<float*>(buf + C::OFF_COL);
    float* sT = reinterpret_cast<float*>(buf + C::OFF_T);
    if (tid < Q) {  // Q is a multiple of 64: whole wavefronts take this branch
      const float lbeg = __shfl(lpre, lane & ~15, 64);  // l at the start of the 16-row tile
      const float lend = __shfl(lpre, lane | 15, 64);   // l at its end
      sL[tid] = lpre;
      sDt[tid] = dpre;
      sRE[tid] = make_float2(__expf(lpre - lbeg), __expf(lpre));
      sCol[tid] = __expf(lend - lpre) * dpre;
    }
    if (tid < R * R) sT[tid] = tt < tr ? __expf(tl1 - tl2) : 0.f;
  };

  if (N < 32) {  // fragment slots past N stay zero for the whole workgroup
    for (int e = tid; e < NTP * NK * 64; e += C::THREADS) {
#pragma unroll
      for (int nb = 0; nb < C::NBUF; ++nb)
        reinterpret_cast<uint4*>(lds + nb * C::BUF + C::OFF_H)[e] = make_uint4(0, 0, 0, 0);
    }
  }
  const int hlast = h0 + HB - 1;
  fetch_head(h0);
  stage_head(lds);
  __syncthreads();

  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    const unsigned char* buf = lds + (C::DB ? (hh & 1) * C::BUF : 0);
    const uint4* sXf = reinterpret_cast<const uint4*>(buf + C::OFF_X);
    const uint4* sHf = reinterpret_cast<const uint4*>(buf + C::OFF_H);
    const float* sL = reinterpret_cast<const float*>(buf + C::OFF_L);
    const float* sDt = reinterpret_cast<const float*>(buf + C::OFF_DT);
    const float2* sRE = reinterpret_cast<const float2*>(buf + C::OFF_RE);
    const float* sCol = reinterpret_cast<const float*>(buf + C::OFF_COL);
    const float* sT = reinterpret_cast<const float*>(buf + C::OFF_T);

    // per-lane decay factors: exp(l_i - l_r0), exp(l_i), and (lanes 16k + t)
    // the tile-boundary factor exp(l_r0 - l_te) of row group k, column tile t
    float rf[RG], el[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const float2 re = sRE[ik[k]];
      rf[k] = re.x;
      el[k] = re.y;
    }
    const int tcol = lane & 15;
    const float tv = lane < 16 * RG && tcol < R ? sT[rk[lane >> 4] * R + tcol] : 0.f;
    auto lanef = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tv), l)); };

    f32x4_t acc[RG][NTP];
    // chunk output: Y^T[p][i] = sum_n Hin[p][n] C_i[n], scaled by exp(l_i)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) {
        const bf16x8_t a = as_bf16x8(sHf[(pt * NK + ks) * 64 + hslot(r16, g4, ks)]);
#pragma unroll
        for (int k = 0; k < RG; ++k)
          acc[k][pt] = mfma_16x16x32(a, Cr[k][ks], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[k][pt]);
      }
    }
#pragma unroll
    for (int k = 0; k < RG; ++k)
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] *= el[k];

    // loads for the next head, in flight during this head's products (the
    // last head re-reads itself, so every iteration has the same sequence of
    // memory operations and the wait before staging covers exactly these
    // loads); issued here rather than at the barrier, where every wavefront
    // would queue its loads at once
    fetch_head(min(h + 1, hlast));

    // intra-chunk, off-diagonal tiles: both row groups walk the same pairs of
    // column tiles (2kp, 2kp+1), so one x fragment feeds both.
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
#pragma unroll
    for (int kp = 0; kp < NM; ++kp) {
      const int ta = 2 * kp, tb = 2 * kp + 1;
      if (ta >= rk[1]) break;  // wavefront-uniform: row group 1 has the most tiles
      // keep each pair's loads next to its products (no hoisting of every
      // pair's operands, which would exhaust the registers)
      __builtin_amdgcn_sched_barrier(0);
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

    // The skip term D_h x_i rides on the diagonal tiles' x operand: an extra
    // product with D_h times the identity, D_h split into two bf16 parts
    // (hi + lo carries 16 bits of D_h; bf16 x times either part is exact in
    // the fp32 accumulator). Lane (i, g4) holds the one identity entry
    // j == i when 4 g4 <= i < 4 g4 + 4.
    const float dh = D != nullptr ? D[h] : 0.f;
    const uint32_t dhi_bits = pack_bf16x2(dh, 0.f) & 0xffffu;
    const uint32_t dlo_bits = pack_bf16x2(dh - bf16_lo(dhi_bits), 0.f) & 0xffffu;
    const int dq = r16 - 4 * g4;
    const bool don = dq >= 0 && dq < 4;
    auto ident = [&](uint32_t bits, bool upper) {
      const uint32_t wv = don ? bits << (16 * (dq & 1)) : 0u;
      const uint32_t w0 = (dq >> 1) == 0 ? wv : 0u, w1 = (dq >> 1) == 1 ? wv : 0u;
      return as_bf16x8(upper ? make_uint4(0, 0, w0, w1) : make_uint4(w0, w1, 0, 0));
    };

    // diagonal tiles: mask (j > i) before the exponential
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const int t = rk[k], i = ik[k];
      const int j0 = 16 * t + 4 * g4;
      const float4 lj = *reinterpret_cast<const float4*>(sL + j0);
      const float4 dj = *reinterpret_cast<const float4*>(sDt + j0);
      const float li = sL[i];
      const float ljv[4] = {lj.x, lj.y, lj.z, lj.w};
      const float djv[4] = {dj.x, dj.y, dj.z, dj.w};
      const uint2 gp = Gd[k];
      const float gv[4] = {bf16_lo(gp.x), bf16_hi(gp.x), bf16_lo(gp.y), bf16_hi(gp.y)};
      float w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jq = j0 + q;
        const float e = __expf(jq <= i ? li - ljv[q] : -INFINITY);
        w[q] = gv[q] * e * djv[q];
      }
      const uint32_t w01 = pack_bf16x2(w[0], w[1]), w23 = pack_bf16x2(w[2], w[3]);
      const bool upper = t & 1;  // which half of the 32-deep pair holds tile t
      const bf16x8_t wop = as_bf16x8(upper ? make_uint4(0, 0, w01, w23) : make_uint4(w01, w23, 0, 0));
      const bf16x8_t dop_hi = ident(dhi_bits, upper), dop_lo = ident(dlo_bits, upper);
      bf16x8_t a[NTP];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) a[pt] = as_bf16x8(xfrag(t >> 1, pt));
      // three rounds over the p tiles, so consecutive products are independent
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(a[pt], wop, acc[k][pt]);
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(a[pt], dop_hi, acc[k][pt]);
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(a[pt], dop_lo, acc[k][pt]);
    }

    // epilogue: store. Rows past the end of the sequence fall outside the
    // buffer range and are dropped, so the store sequence is the same for
    // every chunk.
    uint16_t* ybase = y + (row0 * H + h) * P;
    const __amdgpu_buffer_rsrc_t yr = buffer_range(ybase, (uint32_t)(((rows - 1) * (int64_t)H + 1) * P * 2));
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const uint32_t rowoff = (uint32_t)(ik[k] * (int64_t)H * P * 2);
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) {
        const int p = 16 * pt + 4 * g4;
        const f32x4_t v = acc[k][pt];
        buffer_st8(make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])), yr, rowoff + p * 2);
      }
    }

    // inputs of the next head into the other buffer (nobody reads it during
    // this head)
    if constexpr (!C::DB) __syncthreads();  // one buffer: everyone is done with it
    if (hh + 1 < HB) stage_head(lds + (C::DB ? ((hh + 1) & 1) * C::BUF : 0));
    __syncthreads();
  }
}

// Heads per workgroup: a divisor of the heads in one B/C group, at most 8,
// as large as keeps enough workgroups to fill the chip (the G^T set-up is
// amortised over more heads).
int pick_heads_per_wg(const Plan& p) {
  const int64_t hpg = p.H / p.G;
  const int64_t base = p.batch * p.nc * p.H;
  int hb = 1;
  while (hb < 16 && hpg % (hb * 2) == 0 && base / (hb * 2) >= 256) hb *= 2;
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
      cs, dtc, static_cast<const uint16_t*>(st), static_cast<uint16_t*>(y), p.L, (int)p.H, (int)p.G, p.nc, hb,
      p.ctab);
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
