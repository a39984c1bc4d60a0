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
//  * The R = Q/16 row groups of 16 rows are dealt out in pairs, a short and
//    a long one: wavefront w owns row groups w and R-1-w, w + 1 and R - w
//    causal tiles, R + 1 for every wavefront; with eight wavefronts, the
//    four served first at their SIMDs take one tile more and the other four
//    one tile less (ScanCfg::BAL).
//  * The decay exp(l_i - l_j) is never formed from exp(l_i) * exp(-l_j)
//    (that overflows). Off-diagonal tiles use a factorisation through the
//    tile boundaries, exp(l_i - l_r0) * exp(l_r0 - l_te) * exp(l_te - l_j),
//    r0 the first row of the row group and te the last row of the column
//    tile, every factor <= 1; the three factors are tabulated per head when
//    its inputs are staged. Diagonal tiles are masked (j > i -> 0) before the
//    exponential of l_i - l_j is taken.
//  * Per head, x and Hin are loaded straight from memory into the LDS in
//    their natural row order (loads that write the LDS directly: no
//    registers and no staging instructions), double-buffered: the loads of
//    head h+1 are issued at the start of head h into the other buffer and
//    waited for before the barrier that ends head h. One barrier per head.
//    The matrix-core operands are read from the row-major tiles as they
//    are: Hin fragments (k = n along a row) with 16-byte reads, x fragments
//    (k = j down a column) with the transposing 8-byte LDS read. A per-row
//    XOR of the 16-byte chunk positions keeps both reads free of bank
//    conflicts. The decay tables are tabulated per head from values read
//    into registers.
//  * The skip term D_h x_i shares the diagonal tiles' products: a diagonal
//    tile fills half of a 32-deep step, and the other half carries the bf16
//    part of D_h times the identity against the same x rows; the remainder
//    of D_h is added to the diagonal weight before that is rounded.
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
  // Eight wavefronts (Q = 256) run two per SIMD, wavefront w beside w + 4,
  // and the older one (w < 4) is served first and used to wait at the
  // per-head barrier while its younger neighbour ran alone. The row groups
  // are therefore dealt out unevenly there: the first four wavefronts take
  // the odd row groups (2w + 1, R - 1 - 2w, R + 2 tiles), the last four the
  // even ones (2v, R - 2 - 2v, R tiles), where the one more G^T slot fits
  // the registers. Otherwise: (w, R - 1 - w), R + 1.
  static constexpr bool BAL = WAVES == 8 && N <= 128 && P <= 64;
  static constexpr int NGT = BAL ? R : R - 1;  // off-diagonal G^T slots per wavefront
  // x: Q rows of P bf16, Hin: P rows of N bf16, each in its natural row
  // order with the 16-byte chunks of a row permuted (scan_xsw, scan_hsw); both are
  // filled in 1 KB blocks by loads that write the LDS directly
  static constexpr int XRB = 2 * P, HRB = 2 * N, HCPR = N / 8;
  static constexpr int XBLK = Q * P * 2 / 1024;
  static constexpr int HBLK = (P * N * 2 + 1023) / 1024;
  static constexpr int XBPW = XBLK / WAVES;  // = P / 16
  static constexpr int HBPW = (HBLK + WAVES - 1) / WAVES;
  static constexpr int NSL = (N + 127) / 128;     // n slices when staging B
  static constexpr int NSW = N < 128 ? N : 128;   // width of one slice
  static constexpr int BPITCH = NSW + 8;          // staged B row pitch (bf16)
  // one staging buffer (bytes): x^T fragments, Hin fragments, then per
  // position l, dt, (row factor, exp(l)), column factor, and the R x R
  // table of tile-boundary factors
  static constexpr int X_BYTES = XBLK * 1024;
  static constexpr int H_BYTES = HBLK * 1024;
  static constexpr int OFF_X = 0, OFF_H = X_BYTES, OFF_L = OFF_H + H_BYTES;
  static constexpr int OFF_DT = OFF_L + Q * 4, OFF_RE = OFF_DT + Q * 4;
  static constexpr int OFF_COL = OFF_RE + Q * 8, OFF_T = OFF_COL + Q * 4;
  static constexpr int BUF = OFF_T + R * R * 4;
  static constexpr int BST_BYTES = Q * BPITCH * 2;
  // two buffers when they fit the LDS, else one (and a second barrier per head)
  static constexpr bool DB = 2 * BUF <= 160 * 1024;
  static constexpr int NBUF = DB ? 2 : 1;
  // the B staging area of the G^T set-up lies over buffer 1 when buffer 0
  // and it fit together: then the first head's loads into buffer 0 are
  // issued during the set-up, right after the first B slice's loads
  static constexpr bool EARLY = DB && BUF + BST_BYTES <= 160 * 1024;
  static constexpr int OFF_SB = EARLY ? BUF : 0;
  static constexpr int TOTAL = NBUF * BUF > OFF_SB + BST_BYTES ? NBUF * BUF : OFF_SB + BST_BYTES;
  // read the next pair's operands during the current pair's products where
  // the registers allow it (two operand sets live at once)
  static constexpr bool PIPE = N <= 128 && P <= 64;
};

template <int Q>
constexpr int kScanThreads = 2 * Q;

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

  // row groups of this wavefront, rk[0] < rk[1]
  int rk[RG], ik[RG];
  if constexpr (C::BAL) {
    const int v = wave & 3;
    rk[0] = wave < 4 ? 2 * v + 1 : 2 * v;
    rk[1] = wave < 4 ? R - 1 - 2 * v : R - 2 - 2 * v;
  } else {
    rk[0] = wave;
    rk[1] = R - 1 - wave;
  }
#pragma unroll
  for (int k = 0; k < RG; ++k) ik[k] = 16 * rk[k] + r16;
  // G^T slot of off-diagonal tile t of row group k, static for static k and
  // t: row group 0 fills slots 0.. upwards, row group 1 fills NGT-1..
  // downwards (its tile t at slot NGT-1-t), and as rk[0] + rk[1] <= NGT the
  // two runs meet without overlap.
  auto gslot = [&](int k, int t) {
    const int sidx = k == 0 ? t : C::NGT - 1 - t;
    return sidx < 0 ? 0 : (sidx > C::NGT - 1 ? C::NGT - 1 : sidx);
  };

  // ---- per-head inputs. x and Hin go straight from memory into the LDS (no
  // registers, no staging work): lane l of a 1 KB block fetches the 16-byte
  // chunk that belongs at byte 16 l of the block. Rows of x past the end of
  // the chunk fall outside the buffer range and arrive as zeros. The decay
  // inputs are read into registers and tabulated in the LDS afterwards.
  // Source offsets of the blocks: lane l's chunk of x block k and of Hin
  // block k. With N = 256 they are recomputed at each use from an opaque copy
  // of the lane id instead of held across the head loop: held, they were
  // spilled, and every reload waited for all the loads in flight.
  constexpr bool REMAT = N >= 256 && P <= 64;
  auto xgo_at = [&](int k) {
    int l = lane;
    if constexpr (REMAT) asm volatile("" : "+v"(l));
    const int pos = (wave * C::XBPW + k) * 1024 + 16 * l;
    const int j = pos / C::XRB, cp = (pos % C::XRB) / 16;
    return (uint32_t)(j * H * P * 2 + 16 * (cp ^ scan_xsw<P>(j)));
  };
  auto hgo_at = [&](int k) {
    int l = lane;
    if constexpr (REMAT) asm volatile("" : "+v"(l));
    const int pos = (wave * C::HBPW + k) * 1024 + 16 * l;  // past P*N*2: padding, reads zeros
    const int p = pos / C::HRB, cp = (pos % C::HRB) / 16;
    return (uint32_t)(p * C::HRB + 16 * (cp ^ scan_hsw<N>(p)));
  };
  uint32_t xgo[REMAT ? 1 : C::XBPW], hgo[REMAT ? 1 : C::HBPW];
  if constexpr (!REMAT) {
#pragma unroll
    for (int k = 0; k < C::XBPW; ++k) xgo[k] = xgo_at(k);
#pragma unroll
    for (int k = 0; k < C::HBPW; ++k) hgo[k] = hgo_at(k);
  }
  float lpre = 0.f, dpre = 0.f, tl1 = 0.f, tl2 = 0.f;
  // thread e < R*R tabulates exp(l_{16 r} - l_{16 t + 15}), r = e / R, t = e % R.
  // LDS address of the workgroup's buffer area
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)lds);
  // x block k of this wavefront
  auto fetch_x_block = [&](int h, int bufoff, int k) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + bufoff);
    const v4i32_t xrs = buffer_words(x + (row0 * H + h) * P, (uint32_t)(((rows - 1) * (int64_t)H + 1) * P * 2));
    dma16(xrs, dst + C::OFF_X + (wave * C::XBPW + k) * 1024, REMAT ? xgo_at(k) : xgo[k]);
  };
  // Hin blocks of this wavefront and the decay inputs
  auto fetch_rest = [&](int h, int bufoff) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + bufoff);
    const v4i32_t hrs = buffer_words(states + ((b * H + h) * nc + c) * (int64_t)P * N, (uint32_t)(P * N * 2));
#pragma unroll
    for (int k = 0; k < C::HBPW; ++k)
      if (wave * C::HBPW + k < C::HBLK) dma16(hrs, dst + C::OFF_H + (wave * C::HBPW + k) * 1024, REMAT ? hgo_at(k) : hgo[k]);
    const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
    const float* dc = dtc + ((b * H + h) * nc + c) * Q;
    const int tq = min(tid, Q - 1), te = min(tid, R * R - 1);
    lpre = ld4f_at(lc, 4 * tq);
    dpre = ld4f_at(dc, 4 * tq);
    tl1 = ld4f_at(lc, 64 * (te / R));
    tl2 = ld4f_at(lc, 64 * (te % R) + 60);
  };
  auto fetch_head = [&](int h, int bufoff) {
    fetch_rest(h, bufoff);
#pragma unroll
    for (int k = 0; k < C::XBPW; ++k) fetch_x_block(h, bufoff, k);
  };
  auto stage_tables = [&](unsigned char* buf) {
    const int tr = tid / R, tt = tid % R;
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
  uint16_t* sB = reinterpret_cast<uint16_t*>(lds + C::OFF_SB);
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
    } else {  // (slots between the two runs, if any, repeat a needed tile)
      k = 1;
      t = C::NGT - 1 - e;
    }
    srow[e] = 16 * t + r16;
    sk[e] = k;
  }
  // B is staged one slice of 128 n at a time; each slice's loads are issued
  // before the previous slice's products, and the first head's x and Hin
  // loads after the first slice's, so that the G^T set-up waits for B only.
  constexpr int CH = Q * C::NSW / 8;  // 16-byte chunks of a slice
  constexpr int CPT = (CH + C::THREADS - 1) / C::THREADS;
  uint4 bst[CPT];
  auto load_b = [&](int sl) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ci = min(tid + q * C::THREADS, CH - 1);
      const int j = ci / (C::NSW / 8), n0 = 8 * (ci % (C::NSW / 8));
      bst[q] = ld16_keep(Bm + ((row0 + min(j, rows - 1)) * G + g) * N + sl * 128 + n0, j < rows);
    }
  };
  load_b(0);
#pragma unroll
  for (int sl = 0; sl < C::NSL; ++sl) {
    if (sl > 0) __syncthreads();
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ci = tid + q * C::THREADS;
      if (CH % C::THREADS == 0 || ci < CH) {
        const int j = ci / (C::NSW / 8), n0 = 8 * (ci % (C::NSW / 8));
        st16(sB + j * C::BPITCH + n0, bst[q]);
      }
    }
    if (sl + 1 < C::NSL) load_b(sl + 1);
    if constexpr (C::EARLY) {
      if (sl == 0) fetch_head(h0, 0);
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
  if constexpr (!C::EARLY) {
    __syncthreads();  // the B staging area becomes the head buffers
    fetch_head(h0, 0);
  }
  stage_tables(lds);

  // per-lane LDS byte offsets of the operand reads inside a buffer:
  //  x (A operand X^T, k = j): two transposing reads per fragment, lane
  //  (s, q) = (l % 16, l / 16) addressing row 4q + s / 4 (then 16 rows on),
  //  columns 16 pt + 4 (s % 4) .. +3; the fragment's k order, rows 4q..4q+3
  //  of both 16-row tiles of a 32-row step, is that of the weights below.
  //  Hin (A operand, k = n): row 16 pt + r16, the 16-byte chunk of n = 32 ks + 8 g4.
  int xoff[NTP], hoff[NK];
  {
    const int s = lane & 15, q = lane >> 4;
    const int j = 4 * q + (s >> 2);
#pragma unroll
    for (int pt = 0; pt < NTP; ++pt)
      xoff[pt] = C::OFF_X + j * C::XRB + 16 * ((2 * pt + ((s & 3) >> 1)) ^ scan_xsw<P>(j)) + 8 * (s & 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      hoff[ks] = C::OFF_H + r16 * C::HRB + 16 * (((4 * ks + g4) % C::HCPR) ^ scan_hsw<N>(r16));
  }
  vm_wait<0>();
  __syncthreads();

  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    const unsigned char* buf = lds + (C::DB ? (hh & 1) * C::BUF : 0);
    unsigned char* nbuf = lds + (C::DB ? ((hh + 1) & 1) * C::BUF : 0);
    // loads of the next head into the other buffer, in flight during this
    // head (nobody has read that buffer since the last barrier). They are
    // spread over the head: Hin and the decay inputs now, one x block per
    // step of the off-diagonal loop below. Issued all at once, right after
    // the barrier, the loads of eight wavefronts fill the vector-memory queue
    // and stall every wavefront at the issue.
    const bool pre = C::DB && hh + 1 < HB;
    const int nbo = ((hh + 1) & 1) * C::BUF;
    if (pre) fetch_rest(h + 1, nbo);
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
    auto xfrag = [&](int m, int pt) {
      const unsigned char* a = buf + xoff[pt] + m * 32 * C::XRB;
      const uint2 lo = lds_tr8(a), hi = lds_tr8(a + 16 * C::XRB);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    auto colf = [&](int t) { return *reinterpret_cast<const float4*>(sCol + 16 * t + 4 * g4); };
    // operands of one pair of column tiles (2kp, 2kp + 1): x fragments and
    // the column factors
    struct PairOps {
      uint4 a[NTP];
      float4 ca, cb;
    };
    auto load_pair = [&](int kp, PairOps& o) {
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) o.a[pt] = xfrag(kp, pt);
      o.ca = colf(2 * kp);
      o.cb = colf(2 * kp + 1);
    };

    // chunk output: Y^T[p][i] = sum_n Hin[p][n] C_i[n], scaled by exp(l_i).
    // The fragments of step ks + 1 are read while the products of step ks run.
    {
      uint4 hf[2][NTP];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) hf[0][pt] = ld16(buf + hoff[0] + pt * 16 * C::HRB);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if (ks + 1 < NK) {
#pragma unroll
          for (int pt = 0; pt < NTP; ++pt) hf[(ks + 1) & 1][pt] = ld16(buf + hoff[ks + 1] + pt * 16 * C::HRB);
        }
#pragma unroll
        for (int pt = 0; pt < NTP; ++pt)
#pragma unroll
          for (int k = 0; k < RG; ++k)
            acc[k][pt] = mfma_16x16x32(as_bf16x8(hf[ks & 1][pt]), Cr[k][ks],
                                       ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[k][pt]);
      }
    }
    // the first pair's operands are read while those products drain
    PairOps ops[2];
    load_pair(0, ops[0]);
#pragma unroll
    for (int k = 0; k < RG; ++k)
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] *= el[k];

    // intra-chunk, off-diagonal tiles: both row groups walk the same pairs of
    // column tiles (2kp, 2kp+1), so one x fragment feeds both; the operands
    // of pair kp + 1 are read while pair kp is weighted and multiplied.
    // All factors are <= 1: exp(l_i - l_r0) * exp(l_r0 - l_te) * c_j.
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
      // one pair's products and the next pair's loads per step (no hoisting
      // of every pair's operands, which would exhaust the registers)
      __builtin_amdgcn_sched_barrier(0);
      if (pre && kp < C::XBPW) fetch_x_block(h + 1, nbo, kp);
      if constexpr (C::PIPE) {
        if (kp + 1 < NM) load_pair(kp + 1, ops[(kp + 1) & 1]);
      } else if (kp > 0) {
        load_pair(kp, ops[kp & 1]);
      }
      const PairOps& o = ops[kp & 1];
#pragma unroll
      for (int k = 0; k < RG; ++k) {
        if (ta < rk[k]) {  // tile tb == r_k is the diagonal: excluded here
          const float sa = rf[k] * lanef(16 * k + ta);
          const float sb = tb < rk[k] ? rf[k] * lanef(16 * k + tb) : 0.f;
          const bf16x8_t w = wpair(Gt[gslot(k, ta)], sa, o.ca, Gt[gslot(k, tb)], sb, o.cb);
#pragma unroll
          for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(as_bf16x8(o.a[pt]), w, acc[k][pt]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // x blocks not issued by a wavefront with fewer steps than blocks
    if (pre) {
      const int steps = (rk[1] + 1) / 2;
#pragma unroll
      for (int k = 0; k < C::XBPW; ++k)
        if (k >= steps) fetch_x_block(h + 1, nbo, k);
    }

    // The skip term D_h x_i rides on the diagonal tiles' products. A diagonal
    // tile uses one 16-row half of the 32-deep step, so its x operand holds
    // the tile's rows twice (one transposing read per p tile) and the weight
    // operand's other half holds D_h times the identity. D_h is split into
    // two parts: the bf16 part goes into that identity (bf16 x times it is
    // exact in the fp32 accumulator), the remainder (below 2^-8 |D_h|) onto
    // the diagonal weight before that is rounded, so it adds no error beyond
    // that weight's own rounding. Lane (i, g4) holds the identity entry
    // j == i when 4 g4 <= i < 4 g4 + 4.
    const float dh = D != nullptr ? D[h] : 0.f;
    const uint32_t dhi_bits = pack_bf16x2(dh, 0.f) & 0xffffu;
    const float dlo = dh - bf16_lo(dhi_bits);
    const int dq = r16 - 4 * g4;

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
        w[q] = gv[q] * e * djv[q] + (jq == i ? dlo : 0.f);
      }
      const uint32_t dwv = dq >= 0 && dq < 4 ? dhi_bits << (16 * (dq & 1)) : 0u;
      const bf16x8_t wop = as_bf16x8(make_uint4(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                                                (dq >> 1) == 0 ? dwv : 0u, (dq >> 1) == 1 ? dwv : 0u));
      // rows of tile t: the lower or upper half of its 32-row step
      const unsigned char* xa = buf + (t >> 1) * 32 * C::XRB + (t & 1) * 16 * C::XRB;
      uint2 v[NTP];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) v[pt] = lds_tr8(xa + xoff[pt]);
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt)
        acc[k][pt] = mfma_16x16x32(as_bf16x8(make_uint4(v[pt].x, v[pt].y, v[pt].x, v[pt].y)), wop, acc[k][pt]);
    }

    // this wavefront's loads of the next head have landed (waited for before
    // the stores are issued, so the wait does not include them)
    vm_wait<0>();

    // epilogue: store. Rows past the end of the sequence fall outside the
    // buffer range and are dropped, so the store sequence is the same for
    // every chunk.
    uint16_t* ybase = y + (row0 * H + h) * P;
    const __amdgpu_buffer_rsrc_t yr = buffer_range(ybase, (uint32_t)(((rows - 1) * (int64_t)H + 1) * P * 2));
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const uint32_t rowoff = (uint32_t)(ik[k] * (int64_t)H * P * 2);
      if constexpr (NTP % 2 == 0) {
        // p tiles in pairs: each lane stores eight consecutive p (16 bytes),
        // one store writing 64 contiguous bytes of 16 rows
#pragma unroll
        for (int pt = 0; pt < NTP; pt += 2) {
          const int p = 16 * pt + 16 * (g4 & 1) + 8 * (g4 >> 1);
          buffer_st16(pair_rows16(acc[k][pt], acc[k][pt + 1]), yr, rowoff + p * 2);
        }
      } else {
#pragma unroll
        for (int pt = 0; pt < NTP; ++pt) {
          const int p = 16 * pt + 4 * g4;
          const f32x4_t v = acc[k][pt];
          buffer_st8(make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])), yr, rowoff + p * 2);
        }
      }
    }

    if (hh + 1 < HB) {
      if constexpr (!C::DB) {  // one buffer: refill it once everyone is done with it
        __syncthreads();
        fetch_head(h + 1, 0);
        vm_wait<0>();
      }
      stage_tables(nbuf);
    }
    __syncthreads();
  }
}

// Heads per workgroup: a power-of-two divisor of the heads in one B/C group,
// at most 16, chosen by a small cost model: the workgroups run in rounds of
// `resident` per compute unit, and each costs its heads plus about two heads'
// worth of set-up (the G^T product). More heads per workgroup amortise the
// set-up; fewer avoid a last round that leaves most compute units idle.
// Packed sequences: of the ceil(T/Q) + nseq table slots, about
// ceil(T/Q) + nseq/2 hold tokens (the rest exit at once).
int pick_heads_per_wg(const Plan& p, int resident) {
  const int64_t hpg = p.H / p.G;
  const int64_t used = p.seqtab != nullptr ? p.nc - p.nseq / 2 : p.nc;
  const int64_t units = p.batch * used * p.H;  // (chunk, head) pairs with tokens
  const int64_t slots = (int64_t)device_cu_count() * resident;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int hb = 1; hb <= 16 && hpg % hb == 0; hb *= 2) {
    const int64_t wgs = (units + hb - 1) / hb;
    const int64_t cost = (wgs + slots - 1) / slots * (hb + 2);
    if (cost <= best_cost) {  // ties: the larger count (fewer set-ups)
      best_cost = cost;
      best = hb;
    }
  }
  return best;
}

// The shapes whose register tiles do not fit two wavefronts per SIMD without
// spilling; the plan refuses them (bf16), so they are not instantiated.
template <int P, int N, int Q>
constexpr bool scan_tiles_fit() {
  return !(P == 128 && ((Q == 256 && N >= 64) || (Q == 64 && N == 256))) && !(P == 16 && N == 256 && Q == 256);
}

template <int P, int N, int Q>
hipError_t launch_pnq(const Plan& p, const void* x, const void* B, const void* Cm, const float* D,
                      const float* cs, const float* dtc, const void* st, void* y, hipStream_t s) {
  if constexpr (!scan_tiles_fit<P, N, Q>()) {
    return hipErrorInvalidValue;
  } else {
  using Cfg = ScanCfg<P, N, Q>;
  // workgroups resident per compute unit: two wavefronts per SIMD (the
  // register budget), and the LDS
  const int by_waves = 8 / Cfg::WAVES;
  const int by_lds = 160 * 1024 / Cfg::TOTAL;
  const int hb = pick_heads_per_wg(p, by_waves < by_lds ? by_waves : by_lds);
  const int64_t grid = p.batch * p.nc * (p.H / hb);
  chunk_scan_mfma_kernel<P, N, Q><<<dim3((unsigned)grid), Cfg::THREADS, 0, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(Cm), D,
      cs, dtc, static_cast<const uint16_t*>(st), static_cast<uint16_t*>(y), p.L, (int)p.H, (int)p.G, p.nc, hb,
      p.ctab);
  return hipGetLastError();
  }
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
