// Device helpers shared by the bf16 MFMA kernels (gfx950): buffer resources,
// DMA (global -> LDS) copies, the transposing LDS read, and the LDS layout of
// a 16-byte-chunked tile row.
#pragma once

#include "ra_internal.h"

namespace ra {

typedef __attribute__((address_space(3))) void ra_lds_void;
typedef __attribute__((ext_vector_type(4))) short ra_s16x4;

// Row permutation of a 32-row MFMA A operand: swap bits 2 and 3. With it the
// 16 accumulator registers a lane holds for one 32x32 block are two runs of 8
// consecutive rows (elements 0..7 -> rows 8*hf + 0..7, elements 8..15 -> rows
// 16 + 8*hf + 0..7), which is the k-slot order of the next product's operand.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// LDS layout of a streamed tile of kTileRows rows of up to 128 bf16. The
// tile is cut into 64-column halves, each stored as kTileRows rows of 128
// bytes; 16-byte chunk cc (0..7) of row r of half h sits in slot
// (h * kTileRows + r) * 8 + (cc ^ half_swz(r)).
// The LDS has 64 banks of 4 bytes: two 128-byte rows fill them once, so rows
// of equal parity share banks. A 16-byte read (ds_read_b128) is served 16
// lanes at a time and an 8-byte transposing read 32 lanes at a time; both are
// free of bank conflicts when the lanes served together touch 16 different
// (row parity, chunk) slots.
//  * Row fragments put 16 consecutive rows (a 16-row group in perm_row order)
//    at one chunk in a 16-lane group: half_swz is a bijection on each parity
//    class of a 16-row group.
//  * Column fragments put 4 consecutive rows x 4 consecutive chunks in a
//    32-lane group: half_swz separates rows r and r + 2 by chunk bit 2.
// The swizzle depends only on a row's offset inside a 16-row group and never
// crosses a half, so the half and the 16-row blocks of a fragment read fold
// into the instruction's immediate offset, and each lane keeps only the byte
// offsets of FragOffsets.
constexpr int kTileRows = 64;
__device__ __forceinline__ int half_swz(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
// Slot (16-byte unit) of chunk c (0 .. 15) of tile row r.
__device__ __forceinline__ int tile_slot(int r, int c) {
  return ((c >> 3) * kTileRows + r) * 8 + ((c & 7) ^ half_swz(r));
}
// Inverse: the tile row (in *r) and the chunk of the row held by slot p.
__device__ __forceinline__ int tile_slot_chunk(int p, int* r) {
  *r = (p >> 3) % kTileRows;
  return ((p >> 3) / kTileRows) * 8 + ((p & 7) ^ half_swz(*r));
}

// Per-lane byte offsets of the two fragment kinds the MFMA kernels read.
//  * row[m]: A operand of rows perm_row(lane % 32) of a 32-row block, k-step
//    kk with kk % 4 == m (lane half hf holds chunk 2 * kk + hf). Rows r0 ..
//    r0 + 31 (r0 a multiple of 32), k-step kk: tile + row[kk % 4] +
//    (kk / 4) * kHalfBytes + r0 * 128.
//  * col[half][d1]: transposing read of rows r0 + 8 * hf + 4 * half + i,
//    i = 0..3, columns 32 * dt + 16 * ((lane / 16) % 2) + 4 * (lane % 4) ..
//    + 3 with dt % 2 == d1; rows from r0 (a multiple of 16): tile +
//    col[half][dt % 2] + (dt / 2) * kHalfBytes + r0 * 128.
constexpr int kHalfBytes = kTileRows * 128;
struct FragOffsets {
  uint32_t row[4];
  uint32_t col[2][2];
  __device__ __forceinline__ explicit FragOffsets(int lane) {
    const int l32 = lane & 31, hf = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
    const int pr = perm_row(l32);
#pragma unroll
    for (int m = 0; m < 4; ++m) row[m] = (uint32_t)tile_slot(pr, 2 * m + hf) * 16;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int d1 = 0; d1 < 2; ++d1) {
        const int rl = 8 * hf + 4 * half + (j >> 2);
        const int c = 4 * d1 + 2 * g + ((j & 3) >> 1);
        col[half][d1] = (uint32_t)tile_slot(rl, c) * 16 + 8 * (j & 1);
      }
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// 16-byte load through a buffer resource; offsets past its end read zeros.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16-byte store through a buffer resource; offsets past its end are dropped.
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, float a0, float a1,
                                            float a2, float a3) {
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  u32x4 v = {__float_as_uint(a0), __float_as_uint(a1), __float_as_uint(a2), __float_as_uint(a3)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Number of u in [0, n) for which pred(u) holds, where pred holds on a prefix
// of [0, n) (it is monotone, e.g. a comparison against increasing
// positions). A 64-way search: each round every lane of the (fully active)
// wave probes one evenly spaced u of the remaining range, and the ballot of
// the answers narrows the range to less than the probe spacing, so a range
// of n takes about log64(n) rounds of one load per lane.
template <typename Pred>
__device__ __forceinline__ int prefix_count(int n, int lane, Pred pred) {
  int lo = 0, hi = n;  // the count lies in [lo, hi]
  while (lo < hi) {
    const int step = (hi - lo + 63) >> 6;
    const int p = lo + lane * step;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(p < hi && pred(p)));
    const int nlo = cnt > 0 ? lo + (cnt - 1) * step + 1 : lo;
    hi = min(hi, lo + cnt * step);
    lo = nlo;
  }
  return lo;
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (lds_base is wave-uniform). Issued from inline assembly so that the compiler
// does not track the copy: it would otherwise wait for every copy in flight
// before the next LDS read, including reads of the other buffer. Callers wait
// for completion explicitly (s_waitcnt vmcnt(0)) before the barrier that
// publishes the tile. The LDS address goes in through the "{m0}" operand: the
// compiler itself loads m0 and knows the statement reads it (the statement
// does not write m0). The s_nop separates that write from the copy, which
// reads m0.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ra_lds_void*)lds_base);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(la));
}

// 4 bytes per lane from global memory into LDS at lds_base + 4*lane (issued
// like dma16: untracked by the compiler, awaited explicitly).
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ra_lds_void*)lds_base);
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(la));
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, lane
// j' supplies the address of 4 consecutive bf16; lane j receives element j % 4
// of the rows supplied by lanes 4*i + j/4, i = 0..3. With lane j' pointing at
// T[r0 + j'/4][c0 + 4*(j'%4)], lane j gets T[r0 + i][c0 + j], i = 0..3.
__device__ __forceinline__ uint2 lds_tr4(const void* p) {
  const ra_s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) ra_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(uint2, r);
}

// The row fragment of rows r0 + perm_row(lane % 32), k-step kk (r0 a multiple
// of 32).
__device__ __forceinline__ uint4 tile_row_frag(const uint4* tile, int r0, int kk, const FragOffsets& f) {
  const char* t = reinterpret_cast<const char*>(tile) + (kk >> 2) * kHalfBytes + r0 * 128;
  return *reinterpret_cast<const uint4*>(t + f.row[kk & 3]);
}

// MFMA operand holding T[r0 + 8*hf + i][32*dt + lane%32], i = 0..7: two
// transposing reads (r0 a multiple of 16).
__device__ __forceinline__ uint4 tile_col_frag(const uint4* tile, int r0, int dt, const FragOffsets& f) {
  const char* t = reinterpret_cast<const char*>(tile) + (dt >> 1) * kHalfBytes + r0 * 128;
  const uint2 a0 = lds_tr4(t + f.col[0][dt & 1]);
  const uint2 a1 = lds_tr4(t + f.col[1][dt & 1]);
  return make_uint4(a0.x, a0.y, a1.x, a1.y);
}

}  // namespace ra
