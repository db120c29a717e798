// Pipelined bf16 tile primitives for gfx950 (CDNA4).
//
// Global -> LDS moves use the direct-to-LDS buffer load: each lane loads 16
// bytes, and one wavefront instruction fills 1 KB of LDS at a wave-uniform
// base (lane i lands at base + 16*i).  Buffer resources bound each source, so
// an offset past the buffer (kOOB) reads zeros: padding rows and K/N tails
// need no branches.  Each pipeline stage is its own __shared__ object so the
// compiler tracks the outstanding loads of every stage separately.
//
// Two LDS tile layouts, both in 16-byte chunks with an XOR swizzle that
// spreads the rows a fragment read touches over distinct banks:
//  - K-row tile: row r holds 64 consecutive K values (128 bytes); chunk c of
//    row r sits at r*128 + ((c ^ (r & 7)) * 16).  MFMA fragments are 16-byte
//    reads (8 consecutive K of one row).
//  - N-row tile: row k is one K index holding NCH*8 consecutive M/N values;
//    chunk j of row k sits at k*NCH*16 + ((j ^ swz(k)) * 16).  MFMA fragments
//    come from the transposing LDS read: within each 16-lane group, lane i
//    receives element i%4 of the 8 bytes addressed by lane 4e + i/4 as its
//    e-th value, so 16 lanes addressing a 4 x 16 block receive one column each.
// The MFMA lane mapping matches esg_device.hpp: lane l reads K elements
// kblock*32 + (l/16)*8 + 0..7 of operand row/column l%16.
#pragma once

#include "esg_device.hpp"

#define ESG_LDS __attribute__((address_space(3)))

namespace esg {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kOOB = 0x80000000u;  // at or past every buffer's record count

// Buffer resource over [base, base + bytes); bytes < 2^31 (checked by the host).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Scalar descriptor of a raw (unstrided) buffer for the direct-to-LDS loads:
// base address, record count = `bytes` (offsets at or past it read zero) and
// the same format word as make_rsrc.
struct DmaSrc {
  u32x4_t d;
};
__device__ __forceinline__ DmaSrc make_dma_src(const void* base, uint32_t bytes) {
  const unsigned long long p = (unsigned long long)base;
  DmaSrc s;
  s.d = (u32x4_t){(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)p),
                  (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(p >> 32) & 0xffffu)),
                  (unsigned)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
  return s;
}

// One lane's 16-byte direct-to-LDS load; `wave_base` must be wave-uniform.
// Written as inline assembly on purpose: the compiler then does not treat the
// load as an LDS write, so it adds no waits of its own before LDS reads (it
// cannot tell pipeline stages apart for the transposing reads and would wait
// for every load in flight).  The loads have no register results; the caller
// orders them with explicit vmcnt waits and barriers (wait_vmcnt, barrier).
__device__ __forceinline__ void dma16(const DmaSrc& s, ESG_LDS char* wave_base, uint32_t voff) {
  const int m = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)wave_base);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(s.d), "{m0}"(m) : "memory");
}
// The same with 4 bytes per lane (one wavefront instruction fills 256 bytes).
__device__ __forceinline__ void dma4(const DmaSrc& s, ESG_LDS char* wave_base, uint32_t voff) {
  const int m = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)wave_base);
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(s.d), "{m0}"(m) : "memory");
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// Workgroup barrier without the release fence of __syncthreads (which would
// drain every outstanding direct-to-LDS load); the memory clobber keeps the
// compiler from moving LDS accesses across it.  Callers wait for their own
// loads / LDS reads first.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wave index as a scalar (keeps LDS bases and buffer resources uniform).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// ---- K-row tiles -----------------------------------------------------------
__device__ __forceinline__ int krow_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ uint4 frag_krow(const ESG_LDS char* t, int r, int c) {
  const u32x4_t v = *(const ESG_LDS u32x4_t*)(t + krow_off(r, c));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A second K-row swizzle: chunk c of row r at position c ^ krow_swz2(r), XOR 5
// in rows whose bit 3 is set.  A transposed read (frag_krow_t2) takes rows
// q*8 + 0..3 (q = lane / 16), two adjacent chunks per row; with the plain
// swizzle rows r and r + 8 hit the same banks (2-way conflicts when 32 lanes
// are serviced together), and so do 16 rows read or written along a chunk by
// 16 lanes.  With XOR 5 (bit 0: the 16-row case, bit 2: the chunk pairs of
// the transposed read) a bank model of these accesses finds no conflict for
// groups of 8, 16 or 32 lanes.
__device__ __forceinline__ int krow_swz2(int r) { return (r & 7) ^ (((r >> 3) & 1) * 5); }
__device__ __forceinline__ int krow_off2(int r, int c) { return r * 128 + ((c ^ krow_swz2(r)) << 4); }

__device__ __forceinline__ uint4 frag_krow2(const ESG_LDS char* t, int r, int c) {
  const u32x4_t v = *(const ESG_LDS u32x4_t*)(t + krow_off2(r, c));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 8-byte LDS write of four bf16 (two packed dwords).
__device__ __forceinline__ void lds_write8(ESG_LDS char* p, uint32_t lo, uint32_t hi) {
  *(ESG_LDS u32x2_t*)p = (u32x2_t){lo, hi};
}

// ---- N-row tiles -----------------------------------------------------------
// The transposing read of frag_nrow touches, per 16 lanes, rows 4a..4a+3 of
// one 8-row group and two neighbouring chunks (per 32 lanes: two 8-row groups
// of one 16-row half).  The swizzles below send those (row, chunk) pairs to
// distinct bank groups: rows 0..3 of a group and the group bit 3 select
// distinct even chunk offsets, so the chunk pair stays disjoint too.
template <int NCH>
__device__ __forceinline__ int mn_swz(int k);
template <>
__device__ __forceinline__ int mn_swz<16>(int k) {  // 256-byte rows
  return ((k & 3) << 1) | (((k >> 3) & 1) << 3) | ((k >> 4) & 1);
}
template <>
__device__ __forceinline__ int mn_swz<8>(int k) {  // 128-byte rows: row parity picks the bank half
  return (((k & 1) ^ ((k >> 3) & 1)) << 1) | (((k >> 1) & 1) << 2) | ((k >> 4) & 1);
}
template <>
__device__ __forceinline__ int mn_swz<4>(int k) {  // 64-byte rows: rows k and k+2 (and k+8) share banks
  return (((k >> 1) & 1) ^ ((k >> 3) & 1)) << 1;
}
template <int NCH>
__device__ __forceinline__ int mnrow_off(int k, int j) {
  return k * NCH * 16 + ((j ^ mn_swz<NCH>(k)) << 4);
}

// Fragment of operand columns n0..n0+15 (n0 % 16 == 0) for K-block kb from an
// N-row tile: lane (q = l/16, i = l%16) gets column n0+i at K rows
// kb*32 + q*8 + 0..7.
template <int NCH>
__device__ __forceinline__ uint4 frag_nrow(const ESG_LDS char* t, int kb, int n0, int lane) {
  const int q = lane >> 4, i = lane & 15;
  const int row = kb * 32 + q * 8 + (i >> 2);
  const int colb = n0 * 2 + (i & 3) * 8;  // byte column addressed by this lane
  const int j = colb >> 4, half = colb & 15;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ESG_LDS v4i16*)(t + mnrow_off<NCH>(row, j) + half));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ESG_LDS v4i16*)(t + mnrow_off<NCH>(row + 4, j) + half));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// frag_nrow with the K rows of a 32-row block taken in the order of two
// stacked 16-row accumulator fragments: lane (q = l/16) gets rows
// kb*32 + 4q + 0..3, then kb*32 + 16 + 4q + 0..3.  A B operand built from
// two accumulator fragments of an earlier product (lane q holding their rows
// 4q .. 4q+3) pairs with it element for element, so the product sums the same
// 32 K rows, in another order.
// The tile has 128-byte rows (8 chunks) in its own swizzle, swz_acc8: one
// read instruction touches rows 4q..4q+3 of each lane quarter, i.e. eight
// consecutive rows per 32 lanes, and each needs two neighbouring chunks.  With
// 64 four-byte banks a row's parity picks the bank half, so the chunk pairs of
// the four even (and the four odd) rows of eight must differ, and so must
// those of four consecutive rows (16 lanes at a time): the pair index
// (k & 3) ^ bit 2 of k is a bijection on each of these sets.
__device__ __forceinline__ int swz_acc8(int k) { return ((k & 3) ^ ((k >> 2) & 1)) << 1; }
__device__ __forceinline__ uint4 frag_nrow_acc8(const ESG_LDS char* t, int kb, int n0, int lane) {
  const int q = lane >> 4, i = lane & 15;
  const int row = kb * 32 + q * 4 + (i >> 2);
  const int colb = n0 * 2 + (i & 3) * 8;
  const int j = colb >> 4, half = colb & 15;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (ESG_LDS v4i16*)(t + row * 128 + ((j ^ swz_acc8(row)) << 4) + half));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (ESG_LDS v4i16*)(t + (row + 16) * 128 + ((j ^ swz_acc8(row + 16)) << 4) + half));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// The same transposed fragment (columns m0..m0+15, K rows kb*32 ..) read from
// a K-row tile (128-byte rows, K-row swizzle): the tile's rows are taken as
// the K index and its 64 columns as the M/N index.  Used where one staged
// tile is an operand both along and across its rows.
__device__ __forceinline__ uint4 frag_krow_t(const ESG_LDS char* t, int kb, int m0, int lane) {
  const int q = lane >> 4, i = lane & 15;
  const int row = kb * 32 + q * 8 + (i >> 2);
  const int colb = m0 * 2 + (i & 3) * 8;  // byte column addressed by this lane (within one 16-byte chunk)
  const int c = colb >> 4, half = colb & 15;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ESG_LDS v4i16*)(t + krow_off(row, c) + half));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ESG_LDS v4i16*)(t + krow_off(row + 4, c) + half));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// frag_krow_t on a tile in the second swizzle (krow_off2).
__device__ __forceinline__ uint4 frag_krow_t2(const ESG_LDS char* t, int kb, int m0, int lane) {
  const int q = lane >> 4, i = lane & 15;
  const int row = kb * 32 + q * 8 + (i >> 2);
  const int colb = m0 * 2 + (i & 3) * 8;
  const int c = colb >> 4, half = colb & 15;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ESG_LDS v4i16*)(t + krow_off2(row, c) + half));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ESG_LDS v4i16*)(t + krow_off2(row + 4, c) + half));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

__device__ __forceinline__ void mma_bf16(f32x4& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                               acc, 0, 0, 0);
}

}  // namespace esg
