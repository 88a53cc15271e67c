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

// Chunk swizzle for a tile with 16 chunks of 16 bytes per row that is read
// both by row (one 16-byte chunk per lane, rows perm_row(0..7) together) and
// by the transposing read (4 consecutive rows x 32 bytes per 16-lane group):
// either pattern touches distinct banks.
__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }

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

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (lds_base is wave-uniform). Issued from inline assembly so that the compiler
// does not track the copy: it would otherwise wait for every copy in flight
// before the next LDS read, including reads of the other buffer. Callers wait
// for completion explicitly (s_waitcnt vmcnt(0)) before the barrier that
// publishes the tile.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ra_lds_void*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(la)
               : "m0");
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

// MFMA operand holding T[r0 + 8*hf + i][c0 + lane%32], i = 0..7, from a
// row-major LDS tile of 128-element rows (16 chunks, tile_swz layout).
__device__ __forceinline__ uint4 tile_col_frag(const uint4* tile, int r0, int c0, int lane) {
  const int hf = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
  const int col = c0 + 16 * g + 4 * (j & 3);
  uint2 r2[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = r0 + 8 * hf + 4 * half + (j >> 2);
    const int ch = (col >> 3) ^ tile_swz(r);
    r2[half] = lds_tr4(reinterpret_cast<const char*>(&tile[r * 16 + ch]) + 2 * (col & 7));
  }
  return make_uint4(r2[0].x, r2[0].y, r2[1].x, r2[1].y);
}

// MFMA A operand for rows r0 + perm_row(lane%32) (one 16-byte chunk, k-step kk).
__device__ __forceinline__ uint4 tile_row_frag(const uint4* tile, int r0, int kk, int lane) {
  const int row = r0 + perm_row(lane & 31);
  return tile[row * 16 + ((2 * kk + (lane >> 5)) ^ tile_swz(row))];
}

}  // namespace ra
