// C ABI of the SSD forward pass: argument validation, planning (chunk length,
// workspace carve-up) and the enqueue of the step kernels. Everything up to
// the first launch is plain host code with no HIP call, so the validation is
// testable without a GPU.
#include "../../include/ssd.h"

#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <cstdio>

#include "ssd_internal.h"

namespace ssd {

// (Concurrent first calls on one device store the same value.)
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_chunk_state_simt(const Plan& p, const void* x, const void* B,
                                   const float* dA_cs, const float* dtc, void* states,
                                   hipStream_t s);
hipError_t launch_chunk_scan_simt(const Plan& p, const void* x, const void* B, const void* C,
                                  const float* D, const float* dA_cs, const float* dtc,
                                  const void* states, void* y, hipStream_t s);
bool mfma_chunk_state_supported(const Plan& p);
bool mfma_chunk_scan_supported(const Plan& p);
hipError_t launch_chunk_state_mfma(const Plan& p, const void* x, const void* B,
                                   const float* dA_cs, const float* dtc, void* states,
                                   hipStream_t s);
hipError_t launch_build_chunk_table(const int32_t* cu, int64_t S, int64_t T, int Q, int64_t nslots,
                                    ChunkInfo* tab, int2* seqtab, hipStream_t s);
// steps 1 and 2 in one launch (writes dA_cs and dtc as step 1 does)
hipError_t launch_cumsum_chunk_state_mfma(const Plan& p, const void* x, const void* B, const float* dt,
                                          const float* A, float* dA_cs, float* dtc, void* states,
                                          hipStream_t s);
hipError_t launch_chunk_scan_mfma(const Plan& p, const void* x, const void* B, const void* C,
                                  const float* D, const float* dA_cs, const float* dtc,
                                  const void* states, void* y, hipStream_t s);

namespace {

constexpr size_t kWsAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool is_pow2_in(int64_t v, int64_t lo, int64_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

// Limits keep every grid dimension and every 32-bit in-kernel index in range.
constexpr int64_t kMaxBatch = 65535;
constexpr int64_t kMaxHeads = 65535;
constexpr int64_t kMaxElems = int64_t(1) << 40;

int default_chunk(const ssd_desc_t& d) {
  // 256 halves the chunk-state traffic of 128 (and is faster at every state
  // size up to 256); with headdim 128, and with headdim 16 at dstate 256,
  // the intra-chunk kernel's register tiles only fit at 128.
  if (d.headdim == 16 && d.dstate == 256) return 128;
  return d.headdim <= 64 ? 256 : 128;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

ssd_status_t make_plan(const ssd_desc_t* d, Plan* p) {
  if (d == nullptr || p == nullptr) return SSD_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->headdim <= 0 ||
      d->dstate <= 0 || d->ngroups <= 0)
    return SSD_ERR_BAD_SHAPE;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_BAD_SHAPE;
  if (d->batch > kMaxBatch || d->nheads > kMaxHeads || d->batch * d->nheads > (int64_t(1) << 31))
    return SSD_ERR_BAD_SHAPE;
  if (d->io_dtype != SSD_DTYPE_F32 && d->io_dtype != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
  if (!is_pow2_in(d->headdim, 16, 128)) return SSD_ERR_UNSUPPORTED;
  if (!is_pow2_in(d->dstate, 16, 256)) return SSD_ERR_UNSUPPORTED;
  int Q = d->chunk_size;
  if (Q == 0) Q = default_chunk(*d);
  if (Q != 64 && Q != 128 && Q != 256) return SSD_ERR_UNSUPPORTED;
  // the matrix-core intra-chunk kernel's register tiles do not fit with
  // headdim 128 at chunk length 256 (dstate >= 64) or 64 (dstate 256), nor
  // with headdim 16 at dstate 256 and chunk length 256; those instantiations
  // would spill to scratch, so the combinations are refused
  if (d->io_dtype == SSD_DTYPE_BF16 &&
      ((d->headdim == 128 && ((Q == 256 && d->dstate >= 64) || (Q == 64 && d->dstate == 256))) ||
       (d->headdim == 16 && d->dstate == 256 && Q == 256)))
    return SSD_ERR_UNSUPPORTED;
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  // element counts of the largest arrays must stay well inside 64-bit byte math
  if (d->batch * d->seqlen > kMaxElems / (d->nheads * d->headdim)) return SSD_ERR_BAD_SHAPE;
  if (d->batch * d->nheads * nc > kMaxElems / (d->headdim * d->dstate)) return SSD_ERR_BAD_SHAPE;
  // flattened 1-D grids: (batch * heads * chunks * row blocks) must fit grid.x
  if (d->batch * d->nheads * nc * (Q / 16) >= (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
  p->batch = d->batch;
  p->L = d->seqlen;
  p->H = d->nheads;
  p->P = d->headdim;
  p->N = d->dstate;
  p->G = d->ngroups;
  p->io = d->io_dtype == SSD_DTYPE_BF16 ? kBF16 : kF32;
  p->Q = Q;
  p->nc = nc;
  if (d->dt_clamp && !(d->dt_min <= d->dt_max)) return SSD_ERR_BAD_SHAPE;
  if (!aligned(d->dt_bias, 4)) return SSD_ERR_ALIGNMENT;
  p->dto = DtOpts{d->dt_bias, d->dt_softplus != 0, d->dt_clamp != 0, d->dt_min, d->dt_max};
  return SSD_OK;
}

struct WsLayout {
  size_t cs_off, dt_off, st_off, tab_off, seq_off, total;
  size_t sp_off;  // segmented state passing scratch (0 if not used)
  // one-pass path, inside the states region: the state hand-over ring, then
  // the per-head counters and the ticket (32-bit each)
  size_t ring_off, sync_off;
  int64_t nsync;
  // whole-forward status record (batched layout only): path tag, status bits
  size_t stat_off;
};
constexpr size_t kStatBytes = 256;

// dA_cumsum, dt_chunked, states and (packed sequences) the chunk table, each
// on a kWsAlign boundary. p.nc counts chunk slots. Where the one-pass path
// applies, the states region is large enough for its ring and counters too.
WsLayout ws_layout(const Plan& p, bool with_table = false) {
  WsLayout w;
  const size_t cs_bytes = size_t(p.batch * p.H * p.nc * p.Q) * sizeof(float);
  size_t st_bytes = size_t(p.batch * p.H * p.nc * p.P * p.N) * p.io_bytes();
  w.nsync = p.batch * p.H + 1;
  w.ring_off = 0;
  w.sync_off = 0;
  if (!with_table && fused_forward_supported(p)) {
    const size_t ring = align_up(fused_ring_bytes(p), kWsAlign);
    const size_t need = ring + align_up(size_t(w.nsync) * sizeof(uint32_t), kWsAlign);
    if (need > st_bytes) st_bytes = need;
    w.sync_off = ring;
  }
  w.cs_off = 0;
  w.dt_off = align_up(w.cs_off + cs_bytes, kWsAlign);
  w.st_off = align_up(w.dt_off + cs_bytes, kWsAlign);
  w.ring_off += w.st_off;
  w.sync_off += w.st_off;
  w.tab_off = align_up(w.st_off + st_bytes, kWsAlign);
  w.sp_off = 0;
  if (!with_table && seg_state_passing_applies(p)) {
    w.sp_off = w.tab_off;
    w.tab_off = align_up(w.sp_off + seg_scratch_layout(p, nullptr).bytes, kWsAlign);
  }
  w.seq_off = align_up(w.tab_off + size_t(p.nc) * sizeof(ChunkInfo), kWsAlign);
  w.stat_off = with_table ? 0 : w.tab_off;
  w.total = with_table ? align_up(w.seq_off + size_t(p.nseq) * sizeof(int2), kWsAlign) : w.stat_off + kStatBytes;
  return w;
}

// Packed sequences: the descriptor's batch must be 1 and seqlen the total
// token count T; the chunk slots are ceil(T/Q) + num_seqs (each sequence adds
// at most one partial chunk).
ssd_status_t make_varlen_plan(const ssd_desc_t* d, int64_t num_seqs, Plan* p) {
  ssd_status_t st = make_plan(d, p);
  if (st != SSD_OK) return st;
  if (p->batch != 1 || num_seqs < 1 || num_seqs * p->H >= (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
  if (p->L >= (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;  // token offsets are 32-bit
  const int64_t slots = (p->L + p->Q - 1) / p->Q + num_seqs;
  if (p->H * slots > kMaxElems / (p->P * p->N)) return SSD_ERR_BAD_SHAPE;
  if (p->H * slots * (p->Q / 16) >= (int64_t(1) << 31)) return SSD_ERR_BAD_SHAPE;
  p->nc = slots;
  p->nseq = num_seqs;
  return SSD_OK;
}

// Packed sequences without initial states: fixed chunks of the packed stream
// (the plan of one sequence of T tokens), plus one end window per sequence.
// Workspace: dA_cumsum, dt_chunked, states of the chunks; the segmented
// state-passing scratch where it applies; the per-token sequence-start
// flags; the window table.
struct PackedLayout {
  size_t cs_off, dt_off, st_off, sp_off, seg_off, wtab_off, total;
};
Plan packed_chunk_plan(const Plan& pv) {
  Plan pm = pv;
  pm.nc = (pv.L + pv.Q - 1) / pv.Q;
  pm.ctab = nullptr;
  pm.seqtab = nullptr;
  pm.nseq = 0;
  return pm;
}
PackedLayout packed_layout(const Plan& pm, int64_t S) {
  PackedLayout w;
  const size_t io = pm.io_bytes();
  const size_t cs = size_t(pm.H * pm.nc * pm.Q) * 4, st = size_t(pm.H * pm.nc * pm.P * pm.N) * io;
  w.cs_off = 0;
  w.dt_off = align_up(cs, kWsAlign);
  w.st_off = align_up(w.dt_off + cs, kWsAlign);
  size_t end = align_up(w.st_off + st, kWsAlign);
  w.sp_off = 0;
  if (seg_state_passing_applies(pm)) {
    w.sp_off = end;
    end = align_up(w.sp_off + seg_scratch_layout(pm, nullptr).bytes, kWsAlign);
  }
  w.seg_off = end;
  w.wtab_off = align_up(w.seg_off + size_t(pm.L), kWsAlign);
  w.total = align_up(w.wtab_off + size_t(S) * sizeof(ChunkInfo), kWsAlign);
  return w;
}

// The varlen workspace holds either path's layout (which one runs depends on
// whether initial states are given), then the status record.
struct VarlenLayout {
  WsLayout ws;      // chunks per sequence
  Plan pm;          // fixed chunks of the packed stream
  PackedLayout pl;  // ... and their layout
  size_t stat_off, total;
};
VarlenLayout varlen_layout(const Plan& p, int64_t num_seqs) {
  VarlenLayout v;
  v.ws = ws_layout(p, true);
  v.pm = packed_chunk_plan(p);
  v.pl = packed_layout(v.pm, num_seqs);
  v.stat_off = align_up(v.ws.total > v.pl.total ? v.ws.total : v.pl.total, kWsAlign);
  v.total = v.stat_off + kStatBytes;
  return v;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* ptr, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
  return Range{lo, lo + bytes};
}
bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

ssd_status_t from_hip(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

bool debug_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("SSD_DEBUG");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

// Kernel choice per step. The bf16 io dtype runs the matrix-core kernels; the
// fp32 io dtype keeps fp32 operands and runs the FMA kernels.
hipError_t run_chunk_state(const Plan& p, const void* x, const void* B, const float* cs,
                           const float* dtc, void* st, hipStream_t s) {
  if (mfma_chunk_state_supported(p)) return launch_chunk_state_mfma(p, x, B, cs, dtc, st, s);
  return launch_chunk_state_simt(p, x, B, cs, dtc, st, s);
}
// Steps 1 and 2. bf16: the chunk-state kernel also computes the cumsum of
// its chunk and heads (one launch fewer); fp32: the two stand-alone steps.
hipError_t run_cumsum_chunk_state(const Plan& p, const void* x, const void* B, const float* dt,
                                  const float* A, float* cs, float* dtc, void* st, hipStream_t s) {
  if (mfma_chunk_state_supported(p)) return launch_cumsum_chunk_state_mfma(p, x, B, dt, A, cs, dtc, st, s);
  hipError_t e = launch_chunk_cumsum(p, dt, A, cs, dtc, s);
  if (e == hipSuccess) e = run_chunk_state(p, x, B, cs, dtc, st, s);
  return e;
}
hipError_t run_chunk_scan(const Plan& p, const void* x, const void* B, const void* C,
                          const float* D, const float* cs, const float* dtc, const void* st,
                          void* y, hipStream_t s) {
  if (mfma_chunk_scan_supported(p)) return launch_chunk_scan_mfma(p, x, B, C, D, cs, dtc, st, y, s);
  return launch_chunk_scan_simt(p, x, B, C, D, cs, dtc, st, y, s);
}

// Which path ssd_forward takes: the one-pass kernel where it supports the
// shape and is the faster one for it (fused_forward_preferred), else the
// split path. SSD_FORWARD_PATH=split|fused overrides the choice (fused only
// where supported).
bool use_fused(const Plan& p) {
  if (!fused_forward_supported(p)) return false;
  static const int force = [] {
    const char* v = std::getenv("SSD_FORWARD_PATH");
    if (v == nullptr) return 0;
    if (std::strcmp(v, "split") == 0) return 1;
    if (std::strcmp(v, "fused") == 0) return 2;
    return 0;
  }();
  if (force != 0) return force == 2;
  return fused_forward_preferred(p);
}

// Argument checks shared by the whole-forward entry points (batched layout).
ssd_status_t check_forward(const Plan& p, const void* x, const float* dt, const float* A, const void* B,
                           const void* C, const float* D, const float* init_state, const void* y,
                           const float* final_state, const void* workspace, size_t workspace_bytes,
                           const WsLayout& ws) {
  if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(init_state, 16) ||
      !aligned(final_state, 16) || !aligned(dt, 4) || !aligned(A, 4) || !aligned(D, 4) ||
      !aligned(workspace, kWsAlign))
    return SSD_ERR_ALIGNMENT;
  if (workspace != nullptr && workspace_bytes < ws.total) return SSD_ERR_WORKSPACE;

  const size_t io = p.io_bytes();
  const size_t xy_bytes = size_t(p.batch * p.L * p.H * p.P) * io;
  const size_t bc_bytes = size_t(p.batch * p.L * p.G * p.N) * io;
  const size_t dt_bytes = size_t(p.batch * p.L * p.H) * sizeof(float);
  const size_t hd_bytes = size_t(p.H) * sizeof(float);
  const size_t st_bytes = size_t(p.batch * p.H * p.P * p.N) * sizeof(float);
  const Range in[] = {range_of(x, xy_bytes), range_of(dt, dt_bytes), range_of(A, hd_bytes),
                      range_of(B, bc_bytes), range_of(C, bc_bytes),   range_of(D, hd_bytes),
                      range_of(init_state, st_bytes)};
  const Range ry = range_of(y, xy_bytes);
  const Range rf = range_of(final_state, st_bytes);
  const Range rw = range_of(workspace, ws.total);
  for (const Range& r : in) {
    if (overlap(ry, r)) return SSD_ERR_ALIAS;
    if (overlap(rw, r)) return SSD_ERR_ALIAS;
    // final_state may be exactly init_state (in-place); any other overlap is an error
    if (overlap(rf, r) && !(r.lo == reinterpret_cast<uintptr_t>(init_state) && rf.lo == r.lo)) return SSD_ERR_ALIAS;
  }
  if (overlap(ry, rf) || overlap(ry, rw) || overlap(rf, rw)) return SSD_ERR_ALIAS;
  return SSD_OK;
}

// Enqueue the whole forward on `s` (the workspace allocated in stream order
// when the caller passes none).
ssd_status_t enqueue_forward(const Plan& p, bool fused, const void* x, const float* dt, const float* A,
                             const void* B, const void* C, const float* D, const float* init_state, void* y,
                             float* final_state, void* workspace, const WsLayout& ws, hipStream_t s) {
  void* wbase = workspace;
  bool owned = false;
  if (wbase == nullptr) {
    if (hipMallocAsync(&wbase, ws.total, s) != hipSuccess) return SSD_ERR_HIP;
    owned = true;
  }
  char* w = static_cast<char*>(wbase);
  float* cs = reinterpret_cast<float*>(w + ws.cs_off);
  float* dtc = reinterpret_cast<float*>(w + ws.dt_off);
  void* states = w + ws.st_off;
  if (debug_enabled())
    std::fprintf(stderr, "[ssd] B=%lld L=%lld H=%lld P=%lld N=%lld G=%lld io=%s Q=%d nc=%lld ws=%zu path=%s\n",
                 (long long)p.batch, (long long)p.L, (long long)p.H, (long long)p.P, (long long)p.N,
                 (long long)p.G, p.io == kBF16 ? "bf16" : "fp32", p.Q, (long long)p.nc, ws.total,
                 fused ? "fused" : (mfma_chunk_scan_supported(p) ? "split-mfma" : "split-simt"));
  uint32_t* stat = reinterpret_cast<uint32_t*>(w + ws.stat_off);
  hipError_t e;
  if (fused) {
    uint32_t* sync = reinterpret_cast<uint32_t*>(w + ws.sync_off);
    FusedArgs a{x,    B,       C,  D,   cs, dtc, init_state, y, final_state, reinterpret_cast<float*>(w + ws.ring_off),
                sync, sync + p.batch * p.H, stat + 1};
    e = launch_chunk_cumsum_clear(p, dt, A, cs, dtc, sync, ws.nsync, stat, kPathOnePass, s);
    if (e == hipSuccess) e = launch_fused_forward(p, a, s);
  } else {
    e = run_cumsum_chunk_state(p, x, B, dt, A, cs, dtc, states, s);
    if (e == hipSuccess) {
      if (ws.sp_off != 0)
        e = launch_state_passing_seg(p, states, cs, init_state, final_state, w + ws.sp_off, stat, s);
      else
        e = launch_state_passing(p, states, cs, init_state, final_state, s, stat);
    }
    if (e == hipSuccess) e = run_chunk_scan(p, x, B, C, D, cs, dtc, states, y, s);
  }
  if (e == hipSuccess && debug_enabled()) {
    // check the status record: a bounded wait that was cut off leaves a bit set
    uint32_t rec[2] = {0, 0};
    e = hipMemcpyAsync(rec, stat, sizeof(rec), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess && rec[1] != 0) {
      std::fprintf(stderr, "[ssd] path %u: a bounded wait was cut off (status %u)\n", rec[0], rec[1]);
      e = hipErrorUnknown;
    }
  }
  if (owned) {
    const hipError_t fe = hipFreeAsync(wbase, s);
    if (e == hipSuccess) e = fe;
  }
  return from_hip(e);
}

// Read a status record and, for the paths with bounded waits, check that
// every hand-over happened: stat the record; sync the one-pass counters and
// ticket (nullptr where that path cannot run); seg the segmented
// state-passing scratch (nullptr where it is not laid out).
ssd_status_t read_status(const Plan& p, const char* stat, const char* sync, const char* seg, hipStream_t s,
                         uint32_t* path, uint32_t* status) {
  // Copy n 32-bit words from the workspace and wait for them.
  auto fetch = [&](uint32_t* dst, const void* src, size_t n) {
    hipError_t e = hipMemcpyAsync(dst, src, n * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess;
  };
  // Every word of [src, src + n) equals want(i), read in pieces of kPiece words.
  constexpr int64_t kPiece = 1024;
  uint32_t buf[kPiece];
  bool hip_ok = true;
  auto all_equal = [&](const uint32_t* src, int64_t n, auto want) {
    for (int64_t i0 = 0; i0 < n; i0 += kPiece) {
      const int64_t m = n - i0 < kPiece ? n - i0 : kPiece;
      if (!fetch(buf, src + i0, size_t(m))) {
        hip_ok = false;
        return false;
      }
      for (int64_t i = 0; i < m; ++i)
        if (buf[i] != want(i0 + i)) return false;
    }
    return true;
  };

  uint32_t rec[2] = {0, 0};
  if (!fetch(rec, stat, 2)) return SSD_ERR_HIP;
  uint32_t bits = rec[1] & (SSD_STATUS_WAIT_CUT_OFF_ONE_PASS | SSD_STATUS_WAIT_CUT_OFF_SEGMENTED);
  uint32_t tag = rec[0];
  if (tag == kPathOnePass && sync != nullptr) {
    // every head's counter at its last hand-over, one ticket per workgroup
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(sync);
    const uint32_t last = p.nc > 1 ? uint32_t(p.nc - 1) : 0u;
    const bool flags_ok = all_equal(sw, p.batch * p.H, [&](int64_t) { return last; });
    const uint32_t tickets = uint32_t(fused_forward_grid(p));
    const bool ticket_ok = flags_ok && all_equal(sw + p.batch * p.H, 1, [&](int64_t) { return tickets; });
    if (!flags_ok || !ticket_ok) bits |= SSD_STATUS_CHAIN_INCOMPLETE;
  } else if (tag == kPathSplitSegmented && seg != nullptr) {
    // every segment but the last of each (chain, slice) published, one ticket per workgroup
    const SegScratch sc = seg_scratch_layout(p, const_cast<char*>(seg));
    const int64_t nseg = sc.nseg;
    const bool flags_ok = all_equal(sc.flags, sc.chains * sc.nslice * nseg,
                                    [&](int64_t i) { return (i % nseg) + 1 < nseg ? 1u : 0u; });
    const uint32_t tickets = uint32_t(seg_state_passing_grid(p));
    const bool ticket_ok = flags_ok && all_equal(sc.ticket, 1, [&](int64_t) { return tickets; });
    if (!flags_ok || !ticket_ok) bits |= SSD_STATUS_CHAIN_INCOMPLETE;
  } else if (tag != kPathSplit) {
    tag = SSD_PATH_NONE;
    bits = SSD_STATUS_NO_RECORD;
  }
  if (!hip_ok) return SSD_ERR_HIP;
  if (path != nullptr) *path = tag;
  *status = bits;
  return SSD_OK;
}

}  // namespace
}  // namespace ssd

using ssd::Plan;

extern "C" {

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL_POINTER: return "SSD_ERR_NULL_POINTER: a required pointer is NULL";
    case SSD_ERR_BAD_SHAPE: return "SSD_ERR_BAD_SHAPE: a dimension is <= 0 or too large, or nheads % ngroups != 0";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: headdim, dstate, dtype or chunk size not supported";
    case SSD_ERR_ALIGNMENT: return "SSD_ERR_ALIGNMENT: a base pointer is misaligned";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace smaller than ssd_workspace_bytes()";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: an output overlaps an input";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: the HIP runtime reported an error";
    case SSD_ERR_SCRATCH_LIMIT:
      return "SSD_ERR_SCRATCH_LIMIT: the problem needs more workspace than the 256 MiB no-allocation scratch";
    default: return "unknown ssd_status_t";
  }
}

ssd_status_t ssd_effective_chunk_size(const ssd_desc_t* desc, int32_t* chunk_size) {
  if (chunk_size == nullptr) return SSD_ERR_NULL_POINTER;
  Plan p;
  const ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  *chunk_size = p.Q;
  return SSD_OK;
}

ssd_status_t ssd_workspace_bytes(const ssd_desc_t* desc, size_t* bytes) {
  if (bytes == nullptr) return SSD_ERR_NULL_POINTER;
  Plan p;
  const ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  *bytes = ssd::ws_layout(p).total;
  return SSD_OK;
}

ssd_status_t ssd_forward(const ssd_desc_t* desc, const void* x, const float* dt, const float* A,
                         const void* B, const void* C, const float* D, const float* init_state,
                         void* y, float* final_state, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  const ssd::WsLayout ws = ssd::ws_layout(p);
  st = ssd::check_forward(p, x, dt, A, B, C, D, init_state, y, final_state, workspace, workspace_bytes, ws);
  if (st != SSD_OK) return st;
  return ssd::enqueue_forward(p, ssd::use_fused(p), x, dt, A, B, C, D, init_state, y, final_state, workspace, ws,
                              static_cast<hipStream_t>(stream));
}

ssd_status_t ssd_forward_split(const ssd_desc_t* desc, const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D, const float* init_state,
                               void* y, float* final_state, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  const ssd::WsLayout ws = ssd::ws_layout(p);
  st = ssd::check_forward(p, x, dt, A, B, C, D, init_state, y, final_state, workspace, workspace_bytes, ws);
  if (st != SSD_OK) return st;
  return ssd::enqueue_forward(p, false, x, dt, A, B, C, D, init_state, y, final_state, workspace, ws,
                              static_cast<hipStream_t>(stream));
}

ssd_status_t ssd_forward_fused(const ssd_desc_t* desc, const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D, const float* init_state,
                               void* y, float* final_state, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (!ssd::fused_forward_supported(p)) return SSD_ERR_UNSUPPORTED;
  const ssd::WsLayout ws = ssd::ws_layout(p);
  st = ssd::check_forward(p, x, dt, A, B, C, D, init_state, y, final_state, workspace, workspace_bytes, ws);
  if (st != SSD_OK) return st;
  return ssd::enqueue_forward(p, true, x, dt, A, B, C, D, init_state, y, final_state, workspace, ws,
                              static_cast<hipStream_t>(stream));
}

ssd_status_t ssd_workspace_status(const ssd_desc_t* desc, const void* workspace, size_t workspace_bytes,
                                  void* stream, uint32_t* path, uint32_t* status) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (workspace == nullptr || status == nullptr) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(workspace, ssd::kWsAlign)) return SSD_ERR_ALIGNMENT;
  const ssd::WsLayout ws = ssd::ws_layout(p);
  if (workspace_bytes < ws.total) return SSD_ERR_WORKSPACE;
  const char* w = static_cast<const char*>(workspace);
  return ssd::read_status(p, w + ws.stat_off, ssd::fused_forward_supported(p) ? w + ws.sync_off : nullptr,
                          ws.sp_off != 0 ? w + ws.sp_off : nullptr, static_cast<hipStream_t>(stream), path,
                          status);
}

ssd_status_t ssd_workspace_bytes_varlen(const ssd_desc_t* desc, int64_t num_seqs, size_t* bytes) {
  if (bytes == nullptr) return SSD_ERR_NULL_POINTER;
  Plan p;
  const ssd_status_t st = ssd::make_varlen_plan(desc, num_seqs, &p);
  if (st != SSD_OK) return st;
  *bytes = ssd::varlen_layout(p, num_seqs).total;
  return SSD_OK;
}

ssd_status_t ssd_workspace_status_varlen(const ssd_desc_t* desc, int64_t num_seqs, const void* workspace,
                                         size_t workspace_bytes, void* stream, uint32_t* path, uint32_t* status) {
  Plan p;
  ssd_status_t st = ssd::make_varlen_plan(desc, num_seqs, &p);
  if (st != SSD_OK) return st;
  if (workspace == nullptr || status == nullptr) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(workspace, ssd::kWsAlign)) return SSD_ERR_ALIGNMENT;
  const ssd::VarlenLayout v = ssd::varlen_layout(p, num_seqs);
  if (workspace_bytes < v.total) return SSD_ERR_WORKSPACE;
  const char* w = static_cast<const char*>(workspace);
  return ssd::read_status(v.pm, w + v.stat_off, nullptr, v.pl.sp_off != 0 ? w + v.pl.sp_off : nullptr,
                          static_cast<hipStream_t>(stream), path, status);
}

ssd_status_t ssd_forward_varlen(const ssd_desc_t* desc, const int32_t* cu_seqlens, int64_t num_seqs,
                                const void* x, const float* dt, const float* A, const void* B, const void* C,
                                const float* D, const float* init_states, void* y, float* final_states,
                                void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_varlen_plan(desc, num_seqs, &p);
  if (st != SSD_OK) return st;
  if (!cu_seqlens || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(x, 16) || !ssd::aligned(B, 16) || !ssd::aligned(C, 16) || !ssd::aligned(y, 16) ||
      !ssd::aligned(init_states, 16) || !ssd::aligned(final_states, 16) || !ssd::aligned(dt, 4) ||
      !ssd::aligned(A, 4) || !ssd::aligned(D, 4) || !ssd::aligned(cu_seqlens, 4) ||
      !ssd::aligned(workspace, ssd::kWsAlign))
    return SSD_ERR_ALIGNMENT;
  const ssd::VarlenLayout v = ssd::varlen_layout(p, num_seqs);
  const ssd::WsLayout& ws = v.ws;
  const ssd::PackedLayout& pl = v.pl;
  // bf16 io without initial states: fixed chunks of the packed stream.
  // Otherwise chunks per sequence: each sequence's recurrence starts from its
  // own state, and fp32 io keeps every decay to a few fp32 roundings (in
  // fixed chunks a sequence after k starts in one chunk has its dA cumsum
  // near -128 k, resolved to 2^-16 k)
  const bool fixed_chunks = init_states == nullptr && p.io == ssd::kBF16;
  if (workspace != nullptr && workspace_bytes < v.total) return SSD_ERR_WORKSPACE;

  const size_t io = p.io_bytes();
  const size_t xy_bytes = size_t(p.L * p.H * p.P) * io;
  const size_t bc_bytes = size_t(p.L * p.G * p.N) * io;
  const size_t st_bytes = size_t(num_seqs * p.H * p.P * p.N) * sizeof(float);
  const ssd::Range in[] = {ssd::range_of(x, xy_bytes), ssd::range_of(dt, size_t(p.L * p.H) * sizeof(float)),
                           ssd::range_of(A, size_t(p.H) * sizeof(float)), ssd::range_of(B, bc_bytes),
                           ssd::range_of(C, bc_bytes), ssd::range_of(D, size_t(p.H) * sizeof(float)),
                           ssd::range_of(init_states, st_bytes),
                           ssd::range_of(cu_seqlens, size_t(num_seqs + 1) * sizeof(int32_t))};
  const ssd::Range ry = ssd::range_of(y, xy_bytes);
  const ssd::Range rf = ssd::range_of(final_states, st_bytes);
  const ssd::Range rw = ssd::range_of(workspace, v.total);
  for (const ssd::Range& r : in) {
    if (ssd::overlap(ry, r) || ssd::overlap(rw, r)) return SSD_ERR_ALIAS;
    if (ssd::overlap(rf, r) && !(r.lo == reinterpret_cast<uintptr_t>(init_states) && rf.lo == r.lo))
      return SSD_ERR_ALIAS;
  }
  if (ssd::overlap(ry, rf) || ssd::overlap(ry, rw) || ssd::overlap(rf, rw)) return SSD_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  void* wbase = workspace;
  bool owned = false;
  if (wbase == nullptr) {
    if (hipMallocAsync(&wbase, v.total, s) != hipSuccess) return SSD_ERR_HIP;
    owned = true;
  }
  char* w = static_cast<char*>(wbase);
  uint32_t* stat = reinterpret_cast<uint32_t*>(w + v.stat_off);
  hipError_t e;
  if (fixed_chunks) {
    float* cs = reinterpret_cast<float*>(w + pl.cs_off);
    float* dtc = reinterpret_cast<float*>(w + pl.dt_off);
    void* states = w + pl.st_off;
    uint8_t* seg = reinterpret_cast<uint8_t*>(w + pl.seg_off);
    ssd::ChunkInfo* wtab = reinterpret_cast<ssd::ChunkInfo*>(w + pl.wtab_off);
    Plan pc = v.pm;
    pc.seg_start = seg;
    // the tables kernel also clears the segmented state passing's scratch
    // and writes the status record
    const bool seg_sp = pl.sp_off != 0;
    uint32_t* clr = nullptr;
    int64_t nclr = 0;
    if (seg_sp) {
      const ssd::SegScratch sc = ssd::seg_scratch_layout(pc, w + pl.sp_off);
      clr = sc.flags;
      nclr = sc.nwords;
    }
    e = ssd::launch_build_packed_tables(cu_seqlens, num_seqs, pc.L, pc.Q, seg, wtab, clr, nclr,
                                        seg_sp ? stat : nullptr, ssd::kPathSplitSegmented, s);
    if (e == hipSuccess) e = ssd::run_cumsum_chunk_state(pc, x, B, dt, A, cs, dtc, states, s);
    if (e == hipSuccess) {
      if (seg_sp)
        e = ssd::launch_state_passing_seg(pc, states, cs, nullptr, nullptr, w + pl.sp_off, stat, s, true);
      else
        e = ssd::launch_state_passing(pc, states, cs, nullptr, nullptr, s, stat);
    }
    if (e == hipSuccess) e = ssd::run_chunk_scan(pc, x, B, C, D, cs, dtc, states, y, s);
    if (e == hipSuccess && final_states != nullptr) {
      // the end windows: each one's local state, completed into the final
      // state by the chunk-state kernel itself (bf16 io: the matrix-core kernel)
      Plan pw = pc;
      pw.ctab = wtab;
      pw.nc = num_seqs;
      pw.seg_start = nullptr;  // a window holds one sequence's tokens
      pw.window_finals = final_states;
      pw.window_hin = states;
      pw.window_nc = pc.nc;
      e = ssd::launch_cumsum_chunk_state_mfma(pw, x, B, dt, A, nullptr, nullptr, nullptr, s);
    }
  } else {
    float* cs = reinterpret_cast<float*>(w + ws.cs_off);
    float* dtc = reinterpret_cast<float*>(w + ws.dt_off);
    void* states = w + ws.st_off;
    ssd::ChunkInfo* tab = reinterpret_cast<ssd::ChunkInfo*>(w + ws.tab_off);
    int2* seqtab = reinterpret_cast<int2*>(w + ws.seq_off);
    p.ctab = tab;
    p.seqtab = seqtab;
    e = ssd::launch_build_chunk_table(cu_seqlens, num_seqs, p.L, p.Q, p.nc, tab, seqtab, s);
    if (e == hipSuccess) e = ssd::run_cumsum_chunk_state(p, x, B, dt, A, cs, dtc, states, s);
    if (e == hipSuccess) e = ssd::launch_state_passing(p, states, cs, init_states, final_states, s, stat);
    if (e == hipSuccess) e = ssd::run_chunk_scan(p, x, B, C, D, cs, dtc, states, y, s);
  }
  if (owned) {
    const hipError_t fe = hipFreeAsync(wbase, s);
    if (e == hipSuccess) e = fe;
  }
  return ssd::from_hip(e);
}

ssd_status_t ssd_chunk_cumsum(const ssd_desc_t* desc, const float* dt, const float* A,
                              float* dA_cumsum, float* dt_chunked, void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (!dt || !A || !dA_cumsum || !dt_chunked) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(dt, 4) || !ssd::aligned(A, 4) || !ssd::aligned(dA_cumsum, 16) ||
      !ssd::aligned(dt_chunked, 16))
    return SSD_ERR_ALIGNMENT;
  return ssd::from_hip(
      ssd::launch_chunk_cumsum(p, dt, A, dA_cumsum, dt_chunked, static_cast<hipStream_t>(stream)));
}

ssd_status_t ssd_chunk_state(const ssd_desc_t* desc, const void* x, const void* B,
                             const float* dA_cumsum, const float* dt_chunked, void* states,
                             void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (!x || !B || !dA_cumsum || !dt_chunked || !states) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(x, 16) || !ssd::aligned(B, 16) || !ssd::aligned(dA_cumsum, 16) ||
      !ssd::aligned(dt_chunked, 16) || !ssd::aligned(states, 16))
    return SSD_ERR_ALIGNMENT;
  return ssd::from_hip(ssd::run_chunk_state(p, x, B, dA_cumsum, dt_chunked, states,
                                            static_cast<hipStream_t>(stream)));
}

ssd_status_t ssd_cumsum_chunk_state(const ssd_desc_t* desc, const void* x, const void* B,
                                    const float* dt, const float* A, float* dA_cumsum,
                                    float* dt_chunked, void* states, void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (!x || !B || !dt || !A || !dA_cumsum || !dt_chunked || !states) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(x, 16) || !ssd::aligned(B, 16) || !ssd::aligned(dt, 4) || !ssd::aligned(A, 4) ||
      !ssd::aligned(dA_cumsum, 16) || !ssd::aligned(dt_chunked, 16) || !ssd::aligned(states, 16))
    return SSD_ERR_ALIGNMENT;
  return ssd::from_hip(ssd::run_cumsum_chunk_state(p, x, B, dt, A, dA_cumsum, dt_chunked, states,
                                                   static_cast<hipStream_t>(stream)));
}

ssd_status_t ssd_state_passing(const ssd_desc_t* desc, void* states, const float* dA_cumsum,
                               const float* init_state, float* final_state, void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (!states || !dA_cumsum) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(states, 16) || !ssd::aligned(dA_cumsum, 4) || !ssd::aligned(init_state, 16) ||
      !ssd::aligned(final_state, 16))
    return SSD_ERR_ALIGNMENT;
  const size_t sb = size_t(p.batch * p.H * p.P * p.N) * sizeof(float);
  const ssd::Range rf = ssd::range_of(final_state, sb), ri = ssd::range_of(init_state, sb);
  if (ssd::overlap(rf, ri) && rf.lo != ri.lo) return SSD_ERR_ALIAS;
  return ssd::from_hip(ssd::launch_state_passing(p, states, dA_cumsum, init_state, final_state,
                                                 static_cast<hipStream_t>(stream)));
}

ssd_status_t ssd_chunk_scan(const ssd_desc_t* desc, const void* x, const void* B, const void* C,
                            const float* D, const float* dA_cumsum, const float* dt_chunked,
                            const void* states, void* y, void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (!x || !B || !C || !dA_cumsum || !dt_chunked || !states || !y) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(x, 16) || !ssd::aligned(B, 16) || !ssd::aligned(C, 16) || !ssd::aligned(y, 16) ||
      !ssd::aligned(D, 4) || !ssd::aligned(dA_cumsum, 16) || !ssd::aligned(dt_chunked, 16) ||
      !ssd::aligned(states, 16))
    return SSD_ERR_ALIGNMENT;
  const size_t xy_bytes = size_t(p.batch * p.L * p.H * p.P) * p.io_bytes();
  if (ssd::overlap(ssd::range_of(y, xy_bytes), ssd::range_of(x, xy_bytes))) return SSD_ERR_ALIAS;
  return ssd::from_hip(ssd::run_chunk_scan(p, x, B, C, D, dA_cumsum, dt_chunked, states, y,
                                           static_cast<hipStream_t>(stream)));
}

ssd_status_t ssd_decode_step(const ssd_desc_t* desc, const void* x, const float* dt, const float* A,
                             const void* B, const void* C, const float* D, float* state, void* y,
                             void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (p.L != 1) return SSD_ERR_BAD_SHAPE;
  if (!x || !dt || !A || !B || !C || !state || !y) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(x, 16) || !ssd::aligned(B, 16) || !ssd::aligned(C, 16) || !ssd::aligned(y, 16) ||
      !ssd::aligned(state, 16) || !ssd::aligned(dt, 4) || !ssd::aligned(A, 4) || !ssd::aligned(D, 4))
    return SSD_ERR_ALIGNMENT;
  const size_t io = p.io_bytes();
  const ssd::Range rs = ssd::range_of(state, size_t(p.batch * p.H * p.P * p.N) * sizeof(float));
  const ssd::Range ry = ssd::range_of(y, size_t(p.batch * p.H * p.P) * io);
  const ssd::Range ins[] = {ssd::range_of(x, size_t(p.batch * p.H * p.P) * io),
                            ssd::range_of(dt, size_t(p.batch * p.H) * sizeof(float)),
                            ssd::range_of(A, size_t(p.H) * sizeof(float)),
                            ssd::range_of(B, size_t(p.batch * p.G * p.N) * io),
                            ssd::range_of(C, size_t(p.batch * p.G * p.N) * io),
                            ssd::range_of(D, D ? size_t(p.H) * sizeof(float) : 0)};
  if (ssd::overlap(rs, ry)) return SSD_ERR_ALIAS;
  for (const ssd::Range& r : ins)
    if (ssd::overlap(rs, r) || ssd::overlap(ry, r)) return SSD_ERR_ALIAS;
  return ssd::from_hip(ssd::launch_decode_step(p, x, dt, A, B, C, D, state, y, static_cast<hipStream_t>(stream)));
}

ssd_status_t ssd_conv1d_split(const ssd_desc_t* desc, int32_t conv_width, const void* xbc, const float* weight,
                              const float* bias, int32_t silu, const float* conv_state_in, float* conv_state_out,
                              void* x, void* B, void* C, void* stream) {
  Plan p;
  ssd_status_t st = ssd::make_plan(desc, &p);
  if (st != SSD_OK) return st;
  if (conv_width < 1 || conv_width > 4) return SSD_ERR_UNSUPPORTED;
  if ((p.L + 63) / 64 > 65535) return SSD_ERR_BAD_SHAPE;  // token tiles along grid.y
  if (!xbc || !weight || !x || !B || !C) return SSD_ERR_NULL_POINTER;
  if (!ssd::aligned(xbc, 16) || !ssd::aligned(weight, 4) || !ssd::aligned(bias, 16) ||
      !ssd::aligned(conv_state_in, 4) || !ssd::aligned(conv_state_out, 4) || !ssd::aligned(x, 16) ||
      !ssd::aligned(B, 16) || !ssd::aligned(C, 16))
    return SSD_ERR_ALIGNMENT;
  const size_t io = p.io_bytes();
  const int64_t CH = p.H * p.P + 2 * p.G * p.N;
  const size_t km1 = size_t(conv_width - 1);
  const ssd::Range ins[] = {ssd::range_of(xbc, size_t(p.batch * p.L * CH) * io),
                            ssd::range_of(weight, size_t(CH * conv_width) * sizeof(float)),
                            ssd::range_of(bias, bias ? size_t(CH) * sizeof(float) : 0),
                            ssd::range_of(conv_state_in, conv_state_in ? size_t(p.batch * CH) * km1 * 4 : 0)};
  const ssd::Range outs[] = {ssd::range_of(x, size_t(p.batch * p.L * p.H * p.P) * io),
                             ssd::range_of(B, size_t(p.batch * p.L * p.G * p.N) * io),
                             ssd::range_of(C, size_t(p.batch * p.L * p.G * p.N) * io),
                             ssd::range_of(conv_state_out, conv_state_out ? size_t(p.batch * CH) * km1 * 4 : 0)};
  for (int i = 0; i < 4; ++i) {
    for (const ssd::Range& r : ins)
      if (ssd::overlap(outs[i], r)) return SSD_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (ssd::overlap(outs[i], outs[j])) return SSD_ERR_ALIAS;
  }
  return ssd::from_hip(ssd::launch_conv1d_split(p, conv_width, xbc, weight, bias, silu != 0, conv_state_in,
                                                conv_state_out, x, B, C, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
