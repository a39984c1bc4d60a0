// Steps 2 to 5 in one pass on bf16 matrix cores: the chunk states, the
// recurrence across chunks and the output of every chunk, with each chunk's
// state handed to the next chunk's workgroup instead of making round trips
// through memory between kernels.
//
// The blocked algorithm ("Mamba-2 vs Transformers: SSMs, structured state
// space duality", section "Mamba-2 and the SSD paper: what changed in
// practice") computes a local state per chunk, combines the states with a
// scan over the chunks, and adds each combined state's contribution to its
// chunk's output. For chunk c of head h, with l the within-chunk cumsum of
// dt*A and Lam_c its last entry:
//     S_c   = sum_j exp(Lam_c - l_j) dt_j x_j B_j^T       (chunk state, P x N)
//     H_c   = exp(Lam_c) H_{c-1} + S_c,  H_{-1} = initial state
//     y_i   = sum_{j<=i} exp(l_i - l_j) dt_j (C_i . B_j) x_j
//           + exp(l_i) H_{c-1} C_i + D_h x_i
// Here one workgroup per (chunk, batch, HB heads of one B/C group) computes
// S_c and the intra-chunk output from the x tile it holds in the LDS (x is
// read from memory once), waits until the workgroup of chunk c-1 has
// published H_{c-1} for the head, publishes H_c, and adds the chunk-output
// term. H travels in fp32 through a two-slot ring per (batch, head); the
// last chunk writes it to the final state instead.
//
// Ordering and progress. Workgroups take a ticket from a counter when they
// start and work on the chunk-major item of that ticket, so the producer of
// every state a workgroup waits for holds a smaller ticket: it has started
// and waits only on smaller tickets itself, and every chain drains. The
// states go through loads and stores with device-scope coherence (sc1, the
// encoding device-scope atomics use), and each wavefront waits for its stores
// to complete before the workgroup barrier after which one thread raises the
// head's flag (also a device-scope store). A wait that never ends is cut off
// after a fixed number of polls, with a bit set in the status word, so the
// kernel always exits.
//
// The rest follows the chunk-output kernel: the products are computed
// transposed, Y^T[p][i]; G^T = B C^T is formed once per workgroup and kept
// as packed bf16 in registers; row groups are dealt out in pairs; the decay
// factorisation through tile boundaries keeps every exponent <= 0; x tiles
// are loaded straight into the LDS, double-buffered across heads. B stays in
// the LDS for the whole workgroup: it feeds G^T and, per head, the
// chunk-state product S_c^T = (w o B)^T X with w_j = exp(Lam_c - l_j) dt_j
// (w folded into the B fragments, rounded to bf16; X fragments are those of
// the intra-chunk product).
#include "mfma_common.h"

namespace ssd {
namespace {

// Shapes the kernel is built for: every wavefront gets whole chunk-state
// tiles, and B, the entering state, two x buffers and the tables fit the LDS.
constexpr bool fused_shape_ok(int P, int N, int Q) {
  return P >= 32 && N >= 32 && ((N / 16) * (P / 16)) % (Q / 32) == 0 &&
         Q * 2 * N + P * 2 * N + 2 * (Q * 2 * P + Q * 28 + (Q / 16) * (Q / 16) * 4) <= 160 * 1024;
}

template <int P, int N, int Q>
struct FusedCfg {
  static constexpr int R = Q / 16;            // row groups of 16
  static constexpr int NM = Q / 32;           // 32-deep steps over the chunk positions
  static constexpr int RG = 2;                // row groups per wavefront
  static constexpr int WAVES = R / RG;        // 4 or 8
  static constexpr int THREADS = WAVES * 64;  // = 2 Q
  static constexpr int NTP = P / 16;          // p tiles
  static constexpr int NTN = N / 16;          // n tiles
  static constexpr int NK = N / 32;           // 32-deep steps over n
  // row groups as in the chunk-output kernel: with eight wavefronts the four
  // served first at their SIMDs take one tile more (2w + 1, R - 1 - 2w),
  // the other four one less (2v, R - 2 - 2v), where the registers allow
  static constexpr bool BAL = WAVES == 8 && N <= 128 && P <= 64;
  static constexpr int NGT = BAL ? R : R - 1;  // off-diagonal G^T slots per wavefront
  static constexpr int XRB = 2 * P, HRB = 2 * N, HCPR = N / 8;
  static constexpr int XBLK = Q * P * 2 / 1024, XBPW = XBLK / WAVES;
  static constexpr int BBLK = Q * N * 2 / 1024, BBPW = BBLK / WAVES;
  // chunk-state tiles (n tile, p tile) of one wavefront: SA n tiles by SB p tiles
  static constexpr int SA = NTN >= WAVES ? NTN / WAVES : 1;
  static constexpr int SB = NTN >= WAVES ? NTP : NTP * NTN / WAVES;
  // LDS: B (Q rows of N bf16), the entering state Hin (P rows of N bf16),
  // then two buffers of x (Q rows of P bf16) and the per-head tables
  static constexpr int OFF_B = 0, OFF_HIN = Q * HRB, OFF_BUF = OFF_HIN + P * HRB;
  static constexpr int OFF_X = 0, OFF_L = Q * XRB;
  static constexpr int OFF_DT = OFF_L + Q * 4, OFF_RE = OFF_DT + Q * 4;
  static constexpr int OFF_COL = OFF_RE + Q * 8, OFF_W = OFF_COL + Q * 4, OFF_T = OFF_W + Q * 4;
  static constexpr int BUF = OFF_T + R * R * 4;
  static constexpr int TOTAL = OFF_BUF + 2 * BUF;
  // the ticket is passed to the workgroup through the Hin area, which is
  // first written several barriers later
  static constexpr int OFF_TK = OFF_HIN;
  // read the next pair's operands during the current pair's products where
  // the registers allow it (two operand sets live at once)
  static constexpr bool PIPE = N <= 64;
  static constexpr int YST = RG * NTP / 2;  // y stores per lane and head
  static_assert(N >= 32 && P >= 32, "tile shapes");
  static_assert(TOTAL <= 160 * 1024, "LDS");
  static_assert(fused_shape_ok(P, N, Q), "shape");
  static_assert(XBLK % WAVES == 0 && BBLK % WAVES == 0, "load blocks per wavefront");
  static_assert((NTN * NTP) % WAVES == 0 && SB >= 1 && SA * SB * WAVES == NTN * NTP, "state tiles");
};

constexpr int kSpinLimit = 1 << 18;  // polls of a flag before a wait is given up

template <int P, int N, int Q>
__global__ __launch_bounds__(2 * Q) __attribute__((amdgpu_waves_per_eu(2))) void fused_chunk_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ D, const float* __restrict__ dA_cs, const float* __restrict__ dtc,
    const float* __restrict__ h_init, uint16_t* __restrict__ y, float* __restrict__ h_final,
    float* __restrict__ ring, uint32_t* __restrict__ flags, uint32_t* __restrict__ ticket,
    uint32_t* __restrict__ status, int64_t batch, int64_t L, int H, int G, int64_t nc, int HB) {
  using C = FusedCfg<P, N, Q>;
  constexpr int R = C::R, NM = C::NM, RG = C::RG, NTP = C::NTP, NK = C::NK;
  __shared__ __align__(16) unsigned char lds[C::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int r16 = lane & 15, g4 = lane >> 4;

  // ---- work item of this workgroup's ticket, chunk-major ----
  uint32_t* stk = reinterpret_cast<uint32_t*>(lds + C::OFF_TK);
  if (tid == 0) *stk = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int nhg = H / HB;
  const int64_t tk = __builtin_amdgcn_readfirstlane(*stk);
  const int64_t per_c = batch * nhg;
  if (tk >= per_c * nc) return;  // only if the counter was not cleared (uniform)
  const int64_t c = tk / per_c;
  const int64_t b = (tk - c * per_c) / nhg;
  const int hg = (int)(tk - c * per_c - b * nhg);
  const int h0 = hg * HB;
  const int g = h0 / (H / G);
  const int64_t row0 = b * L + c * Q;
  const int rows = (int)(L - c * Q < Q ? L - c * Q : Q);
  const bool last = c + 1 == nc;

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
  auto gslot = [&](int k, int t) {
    const int sidx = k == 0 ? t : C::NGT - 1 - t;
    return sidx < 0 ? 0 : (sidx > C::NGT - 1 ? C::NGT - 1 : sidx);
  };

  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)lds);

  // ---- B of the chunk and group into the LDS, rows in order, 16-byte
  // chunks permuted by scan_hsw; rows past the end arrive as zeros ----
  {
    const v4i32_t brs = buffer_words(Bm + (row0 * G + g) * N, (uint32_t)(((rows - 1) * (int64_t)G + 1) * N * 2));
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + C::OFF_B);
#pragma unroll
    for (int k = 0; k < C::BBPW; ++k) {
      const int pos = (wave * C::BBPW + k) * 1024 + 16 * lane;
      const int j = pos / C::HRB, cp = (pos % C::HRB) / 16;
      dma16(brs, dst + (wave * C::BBPW + k) * 1024, (uint32_t)(j * G * N * 2 + 16 * (cp ^ scan_hsw<N>(j))));
    }
  }

  // ---- per-head inputs: x into the LDS, decay inputs into registers ----
  uint32_t xgo[C::XBPW];
#pragma unroll
  for (int k = 0; k < C::XBPW; ++k) {
    const int pos = (wave * C::XBPW + k) * 1024 + 16 * lane;
    const int j = pos / C::XRB, cp = (pos % C::XRB) / 16;
    xgo[k] = (uint32_t)(j * H * P * 2 + 16 * (cp ^ scan_xsw<P>(j)));
  }
  float lpre = 0.f, dpre = 0.f, tl1 = 0.f, tl2 = 0.f, lam = 0.f;
  auto fetch_x_block = [&](int h, int bufoff, int k) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + bufoff);
    const v4i32_t xrs = buffer_words(x + (row0 * H + h) * P, (uint32_t)(((rows - 1) * (int64_t)H + 1) * P * 2));
    dma16(xrs, dst + C::OFF_X + (wave * C::XBPW + k) * 1024, xgo[k]);
  };
  auto fetch_rest = [&](int h) {
    const float* lc = dA_cs + ((b * H + h) * nc + c) * Q;
    const float* dc = dtc + ((b * H + h) * nc + c) * Q;
    const int tq = min(tid, Q - 1), te = min(tid, R * R - 1);
    lpre = ld4f_at(lc, 4 * tq);
    dpre = ld4f_at(dc, 4 * tq);
    tl1 = ld4f_at(lc, 64 * (te / R));
    tl2 = ld4f_at(lc, 64 * (te % R) + 60);
    lam = ld4f_at(lc, 4 * (Q - 1));
  };
  auto stage_tables = [&](unsigned char* buf) {
    const int tr = tid / R, tt = tid % R;
    float* sL = reinterpret_cast<float*>(buf + C::OFF_L);
    float* sDt = reinterpret_cast<float*>(buf + C::OFF_DT);
    float2* sRE = reinterpret_cast<float2*>(buf + C::OFF_RE);
    float* sCol = reinterpret_cast<float*>(buf + C::OFF_COL);
    float* sW = reinterpret_cast<float*>(buf + C::OFF_W);
    float* sT = reinterpret_cast<float*>(buf + C::OFF_T);
    if (tid < Q) {  // whole wavefronts
      const float lbeg = __shfl(lpre, lane & ~15, 64);
      const float lend = __shfl(lpre, lane | 15, 64);
      sL[tid] = lpre;
      sDt[tid] = dpre;
      sRE[tid] = make_float2(__expf(lpre - lbeg), __expf(lpre));
      sCol[tid] = __expf(lend - lpre) * dpre;
      sW[tid] = __expf(lam - lpre) * dpre;  // chunk-state weight, <= dt
    }
    if (tid < R * R) sT[tid] = tt < tr ? __expf(tl1 - tl2) : 0.f;
  };
  fetch_rest(h0);
#pragma unroll
  for (int k = 0; k < C::XBPW; ++k) fetch_x_block(h0, C::OFF_BUF, k);

  // ---- C fragments of the row groups (B operand: column i, 8 consecutive n) ----
  bf16x8_t Cr[RG][NK];
  {
    const uint16_t* cbase = Cm + (row0 * G + g) * N;
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const uint32_t coff = (uint32_t)((min(ik[k], rows - 1) * G * N + 8 * g4) * 2);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) Cr[k][ks] = as_bf16x8(ld16_at(cbase, coff + 64 * ks));
    }
  }
  vm_wait<0>();
  __syncthreads();  // B (and the first head's x) in the LDS

  // ---- G^T = B C^T for every tile a row group needs, from the resident B ----
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
      t = C::NGT - 1 - e;
    }
    srow[e] = 16 * t + r16;
    sk[e] = k;
  }
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
    for (int e = 0; e < C::NGT + RG; ++e) {
      const bf16x8_t bfrag = as_bf16x8(
          ld16(lds + C::OFF_B + srow[e] * C::HRB + 16 * ((4 * ks + g4) ^ scan_hsw<N>(srow[e]))));
      const bf16x8_t cfrag = sk[e] == 0 ? Cr[0][ks] : Cr[1][ks];
      Gacc[e] = mfma_16x16x32(bfrag, cfrag, Gacc[e]);
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
  stage_tables(lds + C::OFF_BUF);

  // per-lane LDS byte offsets of the operand reads:
  //  x (X^T fragments, k = j): as in the chunk-output kernel, lane (s, q)
  //  addresses row 4q + s/4 (then 16 rows on), columns 16 pt + 4 (s % 4);
  //  Hin (A operand, k = n): row 16 pt + r16, the 16-byte chunk of n = 32 ks + 8 g4;
  //  B^T fragments of the chunk-state product (k = j): the same transposing
  //  read as x, on the rows of B at the columns of n tile nt.
  const int nt0 = C::NTN >= C::WAVES ? wave * C::SA : wave % C::NTN;
  const int pt0 = C::NTN >= C::WAVES ? 0 : (wave / C::NTN) * C::SB;
  int xoff[NTP], hoff[NK], boff[C::SA];
  {
    const int s = lane & 15, q = lane >> 4;
    const int j = 4 * q + (s >> 2);
#pragma unroll
    for (int pt = 0; pt < NTP; ++pt)
      xoff[pt] = C::OFF_X + j * C::XRB + 16 * ((2 * pt + ((s & 3) >> 1)) ^ scan_xsw<P>(j)) + 8 * (s & 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      hoff[ks] = C::OFF_HIN + r16 * C::HRB + 16 * (((4 * ks + g4) % C::HCPR) ^ scan_hsw<N>(r16));
#pragma unroll
    for (int ni = 0; ni < C::SA; ++ni)
      boff[ni] = C::OFF_B + j * C::HRB + 16 * ((2 * (nt0 + ni) + ((s & 3) >> 1)) ^ scan_hsw<N>(j)) + 8 * (s & 1);
  }
  __syncthreads();

  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    const int64_t bh = b * H + h;
    const unsigned char* buf = lds + C::OFF_BUF + (hh & 1) * C::BUF;
    unsigned char* nbuf = lds + C::OFF_BUF + ((hh + 1) & 1) * C::BUF;
    const bool pre = hh + 1 < HB;
    const int nbo = C::OFF_BUF + ((hh + 1) & 1) * C::BUF;
    if (pre) fetch_rest(h + 1);
    const float* sL = reinterpret_cast<const float*>(buf + C::OFF_L);
    const float* sDt = reinterpret_cast<const float*>(buf + C::OFF_DT);
    const float2* sRE = reinterpret_cast<const float2*>(buf + C::OFF_RE);
    const float* sCol = reinterpret_cast<const float*>(buf + C::OFF_COL);
    const float* sW = reinterpret_cast<const float*>(buf + C::OFF_W);
    const float* sT = reinterpret_cast<const float*>(buf + C::OFF_T);

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
#pragma unroll
    for (int k = 0; k < RG; ++k)
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto xfrag = [&](int m, int pt) {
      const unsigned char* a = buf + xoff[pt] + m * 32 * C::XRB;
      const uint2 lo = lds_tr8(a), hi = lds_tr8(a + 16 * C::XRB);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    auto colf = [&](int t) { return *reinterpret_cast<const float4*>(sCol + 16 * t + 4 * g4); };
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
    PairOps ops[2];
    load_pair(0, ops[0]);

    // ---- intra-chunk, off-diagonal tiles (factors exp(l_i - l_r0) *
    // exp(l_r0 - l_te) * c_j, all <= 1) ----
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
      if (ta >= rk[1]) break;  // wavefront-uniform
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
        if (ta < rk[k]) {
          const float sa = rf[k] * lanef(16 * k + ta);
          const float sb = tb < rk[k] ? rf[k] * lanef(16 * k + tb) : 0.f;
          const bf16x8_t w = wpair(Gt[gslot(k, ta)], sa, o.ca, Gt[gslot(k, tb)], sb, o.cb);
#pragma unroll
          for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(as_bf16x8(o.a[pt]), w, acc[k][pt]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (pre) {
      const int steps = (rk[1] + 1) / 2;
#pragma unroll
      for (int k = 0; k < C::XBPW; ++k)
        if (k >= steps) fetch_x_block(h + 1, nbo, k);
    }

    // ---- diagonal tiles (mask j > i before the exponential) and the skip
    // term D_h x_i in the same products: the x operand holds the tile's rows
    // in both halves of the 32-deep step, the weight operand the masked
    // weights in one half and the bf16 part of D_h times the identity in the
    // other; the remainder of D_h is added to the diagonal weight before that
    // is rounded ----
    const float dh = D != nullptr ? D[h] : 0.f;
    const uint32_t dhi_bits = pack_bf16x2(dh, 0.f) & 0xffffu;
    const float dlo = dh - bf16_lo(dhi_bits);
    const int dq = r16 - 4 * g4;
    const uint32_t dwv = dq >= 0 && dq < 4 ? dhi_bits << (16 * (dq & 1)) : 0u;
    const uint32_t did0 = (dq >> 1) == 0 ? dwv : 0u, did1 = (dq >> 1) == 1 ? dwv : 0u;
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
      const bf16x8_t wop = as_bf16x8(make_uint4(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), did0, did1));
      const unsigned char* xa = buf + (t >> 1) * 32 * C::XRB + (t & 1) * 16 * C::XRB;
      bf16x8_t a[NTP];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) {
        const uint2 v = lds_tr8(xa + xoff[pt]);
        a[pt] = as_bf16x8(make_uint4(v.x, v.y, v.x, v.y));
      }
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) acc[k][pt] = mfma_16x16x32(a[pt], wop, acc[k][pt]);
    }

    // ---- the state chain: Hin = H_{c-1} (the initial state for c = 0), then,
    // once the chunk state below is done, H_c = exp(Lam_c) Hin + S_c. Lane
    // holds Hin[p][n .. n+3] of each of its tiles, p = 16 (pt0 + pi) + r16,
    // n = 16 (nt0 + ni) + 4 g4. The loads are issued before the chunk-state
    // product so that it runs while they are in flight. ----
    f32x4_t hin[C::SA][C::SB];
    // slot tile (ni, pi) of this wavefront: 256 floats, lane l at 4 l
    auto slot_off = [&](int ni, int pi) { return (uint32_t)(((wave * C::SA + ni) * C::SB + pi) * 1024 + 16 * lane); };
    auto nat_off = [&](int ni, int pi) {
      return (int64_t)(16 * (pt0 + pi) + r16) * N + 16 * (nt0 + ni) + 4 * g4;
    };
    if (c == 0) {
#pragma unroll
      for (int ni = 0; ni < C::SA; ++ni)
#pragma unroll
        for (int pi = 0; pi < C::SB; ++pi) {
          if (h_init != nullptr) {
            const float4 v = *reinterpret_cast<const float4*>(h_init + bh * P * N + nat_off(ni, pi));
            hin[ni][pi] = f32x4_t{v.x, v.y, v.z, v.w};
          } else {
            hin[ni][pi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
    } else {
      const uint32_t need = (uint32_t)c;
      for (int spins = 0;; ++spins) {
        const uint32_t v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(flags + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v >= need) break;
        if (spins >= kSpinLimit) {
          if (lane == 0) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      asm volatile("" ::: "memory");  // the state loads stay after the flag
      const __amdgpu_buffer_rsrc_t rs =
          buffer_range(ring + (bh * 2 + ((c - 1) & 1)) * (int64_t)(P * N), (uint32_t)(P * N * 4));
#pragma unroll
      for (int ni = 0; ni < C::SA; ++ni)
#pragma unroll
        for (int pi = 0; pi < C::SB; ++pi) {
          typedef int v4i __attribute__((ext_vector_type(4)));
          const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)slot_off(ni, pi), 0, 16 /* sc1 */);
          hin[ni][pi] = __builtin_bit_cast(f32x4_t, v);
        }
    }
    // ---- chunk state S_c^T[n][p] = sum_j w_j B[j][n] x[j][p]: A operand the
    // weighted B^T fragments (row n, k = j), B operand the x fragments
    // (column p, k = j), both in the k order of the transposing read ----
    f32x4_t sacc[C::SA][C::SB];
#pragma unroll
    for (int ni = 0; ni < C::SA; ++ni)
#pragma unroll
      for (int pi = 0; pi < C::SB; ++pi) sacc[ni][pi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const float4 wa = *reinterpret_cast<const float4*>(sW + 32 * m + 4 * g4);
      const float4 wb = *reinterpret_cast<const float4*>(sW + 32 * m + 16 + 4 * g4);
      uint4 xa[C::SB];
#pragma unroll
      for (int pi = 0; pi < C::SB; ++pi) xa[pi] = xfrag(m, pt0 + pi);
#pragma unroll
      for (int ni = 0; ni < C::SA; ++ni) {
        const unsigned char* a = lds + boff[ni] + m * 32 * C::HRB;
        const uint2 lo = lds_tr8(a), hi = lds_tr8(a + 16 * C::HRB);
        const bf16x8_t bt = as_bf16x8(make_uint4(
            pack_bf16x2(bf16_lo(lo.x) * wa.x, bf16_hi(lo.x) * wa.y), pack_bf16x2(bf16_lo(lo.y) * wa.z, bf16_hi(lo.y) * wa.w),
            pack_bf16x2(bf16_lo(hi.x) * wb.x, bf16_hi(hi.x) * wb.y), pack_bf16x2(bf16_lo(hi.y) * wb.z, bf16_hi(hi.y) * wb.w)));
#pragma unroll
        for (int pi = 0; pi < C::SB; ++pi) sacc[ni][pi] = mfma_16x16x32(bt, as_bf16x8(xa[pi]), sacc[ni][pi]);
      }
    }

    {
      const float eL = __expf(sL[Q - 1]);
      if (!last) {
        const __amdgpu_buffer_rsrc_t ws =
            buffer_range(ring + (bh * 2 + (c & 1)) * (int64_t)(P * N), (uint32_t)(P * N * 4));
#pragma unroll
        for (int ni = 0; ni < C::SA; ++ni)
#pragma unroll
          for (int pi = 0; pi < C::SB; ++pi) {
            typedef int v4i __attribute__((ext_vector_type(4)));
            const f32x4_t hn = hin[ni][pi] * eL + sacc[ni][pi];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, hn), ws, (int)slot_off(ni, pi), 0,
                                                   16 /* sc1 */);
          }
      } else if (h_final != nullptr) {
#pragma unroll
        for (int ni = 0; ni < C::SA; ++ni)
#pragma unroll
          for (int pi = 0; pi < C::SB; ++pi) {
            const f32x4_t hn = hin[ni][pi] * eL + sacc[ni][pi];
            *reinterpret_cast<float4*>(h_final + bh * P * N + nat_off(ni, pi)) = make_float4(hn[0], hn[1], hn[2], hn[3]);
          }
      }
      // Hin as bf16 into the LDS, rows p of N (scan_hsw permutation)
#pragma unroll
      for (int ni = 0; ni < C::SA; ++ni)
#pragma unroll
        for (int pi = 0; pi < C::SB; ++pi) {
          const int p = 16 * (pt0 + pi) + r16;
          const int ch = 2 * (nt0 + ni) + (g4 >> 1);
          *reinterpret_cast<uint2*>(lds + C::OFF_HIN + p * C::HRB + 16 * (ch ^ scan_hsw<N>(p)) + 8 * (g4 & 1)) =
              make_uint2(pack_bf16x2(hin[ni][pi][0], hin[ni][pi][1]), pack_bf16x2(hin[ni][pi][2], hin[ni][pi][3]));
        }
    }
    __syncthreads();  // Hin in the LDS

    // ---- chunk output: Y^T[p][i] += exp(l_i) sum_n Hin[p][n] C_i[n] ----
    {
      f32x4_t acc2[RG][NTP];
      uint4 hf[2][NTP];
#pragma unroll
      for (int pt = 0; pt < NTP; ++pt) hf[0][pt] = ld16(lds + hoff[0] + pt * 16 * C::HRB);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if (ks + 1 < NK) {
#pragma unroll
          for (int pt = 0; pt < NTP; ++pt) hf[(ks + 1) & 1][pt] = ld16(lds + hoff[ks + 1] + pt * 16 * C::HRB);
        }
#pragma unroll
        for (int pt = 0; pt < NTP; ++pt)
#pragma unroll
          for (int k = 0; k < RG; ++k)
            acc2[k][pt] = mfma_16x16x32(as_bf16x8(hf[ks & 1][pt]), Cr[k][ks],
                                        ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc2[k][pt]);
      }
#pragma unroll
      for (int k = 0; k < RG; ++k)
#pragma unroll
        for (int pt = 0; pt < NTP; ++pt) acc[k][pt] += acc2[k][pt] * el[k];
    }

    // ---- store y (rows past the end fall outside the buffer range) ----
    uint16_t* ybase = y + (row0 * H + h) * P;
    const __amdgpu_buffer_rsrc_t yr = buffer_range(ybase, (uint32_t)(((rows - 1) * (int64_t)H + 1) * P * 2));
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      const uint32_t rowoff = (uint32_t)(ik[k] * (int64_t)H * P * 2);
#pragma unroll
      for (int pt = 0; pt < NTP; pt += 2) {
        const int p = 16 * pt + 16 * (g4 & 1) + 8 * (g4 >> 1);
        buffer_st16(pair_rows16(acc[k][pt], acc[k][pt + 1]), yr, rowoff + p * 2);
      }
    }
    if (pre) stage_tables(nbuf);
    // Everything but the y stores just issued has completed: the state
    // stores (vector memory operations complete in issue order) and the
    // loads of the next head. After the barrier every wavefront's part of
    // H_c is in memory and the head's flag is raised.
    asm volatile("" ::: "memory");
    vm_wait<C::YST>();
    __syncthreads();
    if (tid == 0 && !last)
      __hip_atomic_store(flags + bh, (uint32_t)(c + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Heads per workgroup: a power-of-two divisor of the heads in one group, at
// most 16, by the same rounds-times-cost model as the chunk-output kernel.
int pick_fused_heads(const Plan& p, int resident) {
  const int64_t hpg = p.H / p.G;
  const int64_t units = p.batch * p.nc * p.H;
  const int64_t slots = (int64_t)device_cu_count() * resident;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int hb = 1; hb <= 16 && hpg % hb == 0; hb *= 2) {
    const int64_t wgs = (units + hb - 1) / hb;
    const int64_t cost = (wgs + slots - 1) / slots * (hb + 2);
    if (cost <= best_cost) {
      best_cost = cost;
      best = hb;
    }
  }
  return best;
}

template <int P, int N, int Q>
hipError_t launch_fused_pnq(const Plan& p, const FusedArgs& a, hipStream_t s) {
  using Cfg = FusedCfg<P, N, Q>;
  const int by_waves = 8 / Cfg::WAVES;
  const int by_lds = 160 * 1024 / Cfg::TOTAL;
  const int hb = pick_fused_heads(p, by_waves < by_lds ? by_waves : by_lds);
  const int64_t grid = p.batch * p.nc * (p.H / hb);
  fused_chunk_mfma_kernel<P, N, Q><<<dim3((unsigned)grid), Cfg::THREADS, 0, s>>>(
      static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C), a.D,
      a.dA_cs, a.dtc, a.h_init, static_cast<uint16_t*>(a.y), a.h_final, a.ring, a.flags, a.ticket, a.status,
      p.batch, p.L, (int)p.H, (int)p.G, p.nc, hb);
  return hipGetLastError();
}

template <int P, int N>
hipError_t launch_fused_pn(const Plan& p, const FusedArgs& a, hipStream_t s) {
  if constexpr (fused_shape_ok(P, N, 256)) return launch_fused_pnq<P, N, 256>(p, a, s);
  return hipErrorInvalidValue;
}

template <int P>
hipError_t launch_fused_p(const Plan& p, const FusedArgs& a, hipStream_t s) {
  switch (p.N) {
    case 32: return launch_fused_pn<P, 32>(p, a, s);
    case 64: return launch_fused_pn<P, 64>(p, a, s);
    case 128: return launch_fused_pn<P, 128>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fused_forward_supported(const Plan& p) {
  if (p.io != kBF16 || p.ctab != nullptr || p.Q != 256) return false;
  if (!(p.P == 32 || p.P == 64) || !(p.N == 32 || p.N == 64 || p.N == 128)) return false;
  if (!fused_shape_ok((int)p.P, (int)p.N, p.Q)) return false;
  // 32-bit byte offsets inside one chunk's rows of x, y and B
  if (int64_t(p.Q) * p.H * p.P * 2 >= (int64_t(1) << 31)) return false;
  if (int64_t(p.Q) * p.G * p.N * 2 >= (int64_t(1) << 31)) return false;
  return true;
}

namespace {
// workgroups resident per compute unit and heads per workgroup of the launch
template <int P, int N, int Q>
void fused_launch_shape(const Plan& p, int& resident, int& hb) {
  using Cfg = FusedCfg<P, N, Q>;
  const int by_waves = 8 / Cfg::WAVES;
  const int by_lds = 160 * 1024 / Cfg::TOTAL;
  resident = by_waves < by_lds ? by_waves : by_lds;
  hb = pick_fused_heads(p, resident);
}
template <int P>
bool fused_shape_of(const Plan& p, int& resident, int& hb) {
  switch (p.N) {
    case 32: if constexpr (fused_shape_ok(P, 32, 256)) { fused_launch_shape<P, 32, 256>(p, resident, hb); return true; } break;
    case 64: if constexpr (fused_shape_ok(P, 64, 256)) { fused_launch_shape<P, 64, 256>(p, resident, hb); return true; } break;
    case 128: if constexpr (fused_shape_ok(P, 128, 256)) { fused_launch_shape<P, 128, 256>(p, resident, hb); return true; } break;
  }
  return false;
}
}  // namespace

// The one-pass kernel pays for its chains once per round of workgroups: the
// last chunk's workgroup of a chain first waits for nc - 1 hand-overs (a few
// microseconds each). It saves the second read of x and the state round trips
// on every head-chunk. Measured on MI355X: it is ahead once the work takes at
// least two rounds of workgroups with chains of at most 16 chunks, and behind
// with one round (the hand-overs not amortised) or longer chains.
bool fused_forward_preferred(const Plan& p) {
  if (!fused_forward_supported(p) || p.nc > 16) return false;
  int resident = 1, hb = 1;
  const bool ok = p.P == 32 ? fused_shape_of<32>(p, resident, hb) : fused_shape_of<64>(p, resident, hb);
  if (!ok) return false;
  const int64_t wgs = p.batch * p.nc * (p.H / hb);
  const int64_t slots = (int64_t)device_cu_count() * resident;
  return wgs >= 2 * slots;
}

int64_t fused_forward_grid(const Plan& p) {
  int resident = 1, hb = 1;
  const bool ok = p.P == 32 ? fused_shape_of<32>(p, resident, hb) : fused_shape_of<64>(p, resident, hb);
  return ok ? p.batch * p.nc * (p.H / hb) : 0;
}

size_t fused_ring_bytes(const Plan& p) { return size_t(p.batch * p.H * 2) * size_t(p.P * p.N) * sizeof(float); }

hipError_t launch_fused_forward(const Plan& p, const FusedArgs& a, hipStream_t s) {
  switch (p.P) {
    case 32: return launch_fused_p<32>(p, a, s);
    case 64: return launch_fused_p<64>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
