// gfx950 matrix-core helpers shared by the bf16 contraction kernels.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (D[16x16] += A[16x32] B[32x16]),
// with lane l = 16*g + r (g = l / 16 in 0..3, r = l % 16):
//   A: lane holds A[r][8g .. 8g+7]      (row r, eight consecutive k)
//   B: lane holds B[8g .. 8g+7][r]      (column r, eight consecutive k)
//   D: lane holds D[4g + i][r], i = 0..3 (four consecutive rows of column r)
// Only the pairing of k between A and B matters for the product, so any
// permutation of the 32 k indices may be used as long as A and B agree.
#pragma once

#include "ssd_internal.h"

namespace ssd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ f32x4_t mfma_16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                 const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(const bf16x8_t& v) { return v; }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Load 16 bytes from an address that is always valid (the caller clamps it)
// and keep them only when `keep` holds. Unlike `keep ? ld16(p) : 0` this is
// branch-free, so many such loads can be in flight at once.
__device__ __forceinline__ uint4 ld16_keep(const void* p, bool keep) {
  const uint4 v = ld16(p);
  return keep ? v : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Loads at a wavefront-uniform base plus a 32-bit per-lane byte offset: the
// address takes one vector register (scalar base + vector offset) instead of
// a 64-bit pointer per lane.
__device__ __forceinline__ uint4 ld16_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(base) + byte_off);
}
__device__ __forceinline__ float ld4f_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(base) + byte_off);
}

// A raw buffer resource covering [base, base + bytes): stores at offsets at or
// past `bytes` are discarded by the hardware's range check. This lets a
// ragged tail be written with the same unconditional store sequence as a full
// tile (no divergent branch around the stores).
// `base` and `bytes` must be the same in every lane of the wavefront: they
// are read from the first active lane, which keeps the descriptor in scalar
// registers (otherwise every store becomes a loop over distinct descriptors).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ void buffer_st8(const uint2& v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(v2i{(int)v.x, (int)v.y}, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buffer_st16(const uint4& v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, r, (int)off, 0, 0);
}

// Two accumulator tiles of a 16x16 product (lane row g = l / 16 holding rows
// 4g..4g+3 of column l % 16 in each) as bf16, rearranged so that each lane
// holds eight consecutive rows of one tile pair: rows 1 and 3 of lanes (16
// lanes each) of the first tile trade places with rows 0 and 2 of the
// second. Lane row g then holds rows 16 (g & 1) + 8 (g >> 1) .. +7 of the
// 32 rows of the pair (first tile rows 0..15, second 16..31), in order.
__device__ __forceinline__ uint4 pair_rows16(const f32x4_t& t0, const f32x4_t& t1) {
  const auto s0 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(t0[0], t0[1]), pack_bf16x2(t1[0], t1[1]), false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(t0[2], t0[3]), pack_bf16x2(t1[2], t1[3]), false, false);
  return make_uint4(s0[0], s1[0], s0[1], s1[1]);
}

// XOR of one constant per set bit of r mod 16 (m0 for bit 0, ...): the
// row-dependent chunk permutation of tiles staged in the LDS.
__device__ __forceinline__ constexpr int row_xor(int r, int m0, int m1, int m2, int m3) {
  return ((r & 1) ? m0 : 0) ^ ((r & 2) ? m1 : 0) ^ ((r & 4) ? m2 : 0) ^ ((r & 8) ? m3 : 0);
}

// Chunk permutations of tiles staged row by row in the LDS for the chunk
// output kernels: row r's 16-byte chunk c is stored at chunk position
// c ^ sw(r), sw(r) the XOR of one constant per set bit of r mod 16
// (row_xor). The constants keep the operand reads free of bank conflicts on
// gfx950 (64 banks of 4 bytes): the transposing 8-byte read of x rows covers
// four consecutive rows and two adjacent chunks per 16 lanes; the 16-byte
// read of rows of N bf16 (the entering state, B) serves its eight-lane groups
// in the pairs (0-7, 24-31), (8-15, 16-23), ... (as measured), each pair
// reading eight consecutive rows at the chunk of one lane group and eight
// rows at the next chunk.
template <int P>
__device__ __forceinline__ int scan_xsw(int j) {  // rows of P bf16 (x)
  return P == 32 ? row_xor(j, 0, 2, 2, 0) : P == 64 ? row_xor(j, 2, 4, 2, 0) : P == 128 ? row_xor(j, 2, 4, 8, 0) : 0;
}
template <int N>
__device__ __forceinline__ int scan_hsw(int p) {  // rows of N bf16 (Hin, B)
  return N == 16 ? 0 : N == 32 ? row_xor(p, 0, 0, 1, 2) : N == 64 ? row_xor(p, 0, 1, 2, 4) : row_xor(p, 1, 2, 4, 8);
}

// A raw buffer descriptor over [base, base + bytes) as four scalar words
// (base and bytes wavefront-uniform).
typedef int v4i32_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i32_t buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i32_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)a), (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)),
                 (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// 16 bytes per lane from a buffer straight into the LDS: lane l's bytes land
// at LDS address lds_dst + 16 l (lds_dst wavefront-uniform); offsets past the
// buffer's range read zeros. Written as inline assembly so that the compiler
// does not treat it as a write to every LDS buffer (it would then wait for
// the load before the next LDS read of the other buffer): completion is
// waited for explicitly (vm_wait) before the barrier that publishes the
// buffer. No result registers; the address register is read at issue.
// The load takes its LDS address from m0, which the compiler reserves but
// does not otherwise use in these kernels (no other LDS-DMA, interpolation or
// indexed-register instructions), so nothing it holds there is lost.
// (The clobber of m0 is the point: the compiler is told the register changes.
// It warns that m0 is reserved; that warning is expected here.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const v4i32_t& r, uint32_t lds_dst, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(voff), "s"(__builtin_bit_cast(__int128, r))
               : "memory", "m0");
}
#pragma clang diagnostic pop

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Transposing 8-byte LDS read (16-bit elements): within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces addressed by
// lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4, in that order. With lane
// s addressing row s / 4 (of four consecutive rows) at column 4 (s % 4), lane
// i receives column i of the four rows: a matrix-core operand fragment whose
// k runs along the rows.
__device__ __forceinline__ uint2 lds_tr8(const unsigned char* p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
  return __builtin_bit_cast(uint2, v);
}

// Wait until at most n vector memory operations of this wavefront are in
// flight (loads into the LDS included); other counters are not waited for.
template <int n>
__device__ __forceinline__ void vm_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroups are handed to the eight XCDs (each with its own L2) round-robin
// by workgroup id. This renumbering gives each XCD one contiguous run of
// logical ids, so workgroups that share operands (neighbouring logical ids:
// the heads of one chunk) run on the same XCD and meet in its L2.
__device__ __forceinline__ int64_t xcd_local_order(int64_t bid, int64_t grid) {
  constexpr int kXcds = 8;
  if (grid % kXcds != 0) return bid;
  return (bid % kXcds) * (grid / kXcds) + bid / kXcds;
}

// Element e (0..7) of a row of eight bf16 held in a uint4, as fp32.
__device__ __forceinline__ float bf16_at(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

}  // namespace ssd
