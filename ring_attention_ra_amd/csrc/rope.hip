// Rotary position embedding (intelliparadigm.com long-context survey, §2.1.3
// RoPE的旋转位置编码): element j of a row's first half and element j of its
// second half form a pair, turned by the angle pos * base^(-2j/d).
//
// The pass is memory-bound (one read and one write of the tensor), and it runs
// once per chunk: a K tile is read by every query block of a step, so turning
// K once in HBM costs far less than turning it inside the attention loop.
//  * Each thread owns VEC consecutive pairs of a row: VEC elements from each
//    half, so the 16 lanes serving a 128-wide bf16 row read and write two
//    contiguous 128-byte runs.
//  * The angle is formed as a fraction of a turn in double precision
//    (position times frequency / 2 pi, minus the nearest integer), so positions
//    up to 2^31 keep full accuracy; sine and cosine come from the hardware
//    instructions, which take a fraction of a turn, and the rotation runs in fp32.
//  * The threads of a block keep the same pairs of every row they visit (the
//    block size is a multiple of the pairs per row when the fast path is taken),
//    so the frequencies are formed once per thread.
#include <algorithm>
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

// VEC consecutive elements to / from fp32: one 8-byte (bf16) or 16-byte (fp32)
// access when VEC is 4 (the caller guarantees the alignment), else one each.
template <int VEC>
__device__ __forceinline__ void load_vec(const uint16_t* p, float (&f)[VEC]) {
  if constexpr (VEC == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    for (int v = 0; v < VEC; ++v) f[v] = __uint_as_float((uint32_t)p[v] << 16);
  }
}
template <int VEC>
__device__ __forceinline__ void load_vec(const float* p, float (&f)[VEC]) {
  if constexpr (VEC == 4) {
    const float4 w = *reinterpret_cast<const float4*>(p);
    f[0] = w.x, f[1] = w.y, f[2] = w.z, f[3] = w.w;
  } else {
    for (int v = 0; v < VEC; ++v) f[v] = p[v];
  }
}
template <int VEC>
__device__ __forceinline__ void store_vec(uint16_t* p, const float (&f)[VEC]) {
  if constexpr (VEC == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(ra_pack_bf16(f[0], f[1]), ra_pack_bf16(f[2], f[3]));
  } else {
    for (int v = 0; v < VEC; ++v) p[v] = (uint16_t)(ra_pack_bf16(f[v], 0.0f) & 0xffffu);
  }
}
template <int VEC>
__device__ __forceinline__ void store_vec(float* p, const float (&f)[VEC]) {
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  } else {
    for (int v = 0; v < VEC; ++v) p[v] = f[v];
  }
}

// Turn the loaded pairs by p * turns and store them at y + base (first half)
// and y + base + half (second half).
template <typename T, int VEC>
__device__ __forceinline__ void rotate_store(T* y, int64_t base, int half, double p, const double (&turns)[VEC],
                                             const float (&x1)[VEC], const float (&x2)[VEC]) {
  float y1[VEC], y2[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const double t = p * turns[v];
    const float frac = (float)(t - rint(t));  // in [-1/2, 1/2] turn
    // v_sin_f32 / v_cos_f32 take their argument in turns.
    const float s = __builtin_amdgcn_sinf(frac), c = __builtin_amdgcn_cosf(frac);
    y1[v] = x1[v] * c - x2[v] * s;
    y2[v] = x1[v] * s + x2[v] * c;
  }
  store_vec<VEC>(y + base, y1);
  store_vec<VEC>(y + base + half, y2);
}

// Pair group g (pairs VEC*g .. VEC*g + VEC - 1) of row `row` (position pos).
template <typename T, int VEC>
__device__ __forceinline__ void rotate_group(const T* x, T* y, int64_t row, int64_t len, int d,
                                             int g, const int32_t* pos, const double (&turns)[VEC]) {
  const int half = d >> 1;
  const int64_t base = row * d + (int64_t)VEC * g;
  const double p = (double)pos[row % len];
  float x1[VEC], x2[VEC];
  load_vec<VEC>(x + base, x1);
  load_vec<VEC>(x + base + half, x2);
  rotate_store<T, VEC>(y, base, half, p, turns, x1, x2);
}

// turns_j = base^(-2j/d) / (2 pi): the angle per position in turns.
__device__ __forceinline__ double turns_of(int j, int d, double log2_base) {
  return exp2(-2.0 * (double)j / (double)d * log2_base) * 0.15915494309189533577;
}

template <typename T, int VEC>
__global__ void rope_kernel(const T* x, T* y, const int32_t* __restrict__ pos, int64_t rows, int64_t len,
                            int d, double log2_base, int fixed_group) {
  const int groups = (d >> 1) / VEC;
  const int64_t total = rows * groups;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (fixed_group) {  // blockDim.x and the grid stride are multiples of `groups`
    const int g = (int)(threadIdx.x % groups);
    double turns[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) turns[v] = turns_of(VEC * g + v, d, log2_base);
    // Four rows per trip, loads first, so that each thread has more bytes in
    // flight (each thread only ever touches its own elements, so this is safe
    // in place too).
    for (; i + 3 * stride < total; i += 4 * stride) {
      float x1[4][VEC], x2[4][VEC];
      int64_t base[4];
      double p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = (i + u * stride) / groups;
        base[u] = row * d + (int64_t)VEC * g;
        p[u] = (double)pos[row % len];
        load_vec<VEC>(x + base[u], x1[u]);
        load_vec<VEC>(x + base[u] + (d >> 1), x2[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) rotate_store<T, VEC>(y, base[u], d >> 1, p[u], turns, x1[u], x2[u]);
    }
    for (; i < total; i += stride) rotate_group<T, VEC>(x, y, i / groups, len, d, g, pos, turns);
  } else {
    for (; i < total; i += stride) {
      const int g = (int)(i % groups);
      double turns[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) turns[v] = turns_of(VEC * g + v, d, log2_base);
      rotate_group<T, VEC>(x, y, i / groups, len, d, g, pos, turns);
    }
  }
}

template <typename T, int VEC>
hipError_t launch_rope_t(const void* x, void* y, const int32_t* pos, int64_t rows, int64_t len, int d,
                         double log2_base, hipStream_t stream) {
  const int groups = (d >> 1) / VEC;
  const int threads = 256;
  const int fixed = threads % groups == 0 ? 1 : 0;
  // Four rows per thread where the groups fit a block evenly: the kernel's
  // batched trip then runs, and each thread's angle setup serves four rows.
  const int64_t per_thread = fixed ? 4 : 1;
  int64_t blocks = (rows * groups + threads * per_thread - 1) / (threads * per_thread);
  blocks = std::max<int64_t>(1, std::min<int64_t>(blocks, 256 * 64));
  hipLaunchKernelGGL((rope_kernel<T, VEC>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const T*>(x), static_cast<T*>(y), pos, rows, len, d, log2_base, fixed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t outer, int64_t len, int32_t d,
                       int32_t dtype, float base, hipStream_t stream) {
  const int64_t rows = outer * len;
  const double l2b = std::log2((double)base);
  const uintptr_t align = (uintptr_t)x | (uintptr_t)y;
  const bool vec4 = ((d >> 1) % 4) == 0 && align % (dtype == RA_BF16 ? 8 : 16) == 0;
  if (dtype == RA_BF16)
    return vec4 ? launch_rope_t<uint16_t, 4>(x, y, pos, rows, len, d, l2b, stream)
                : launch_rope_t<uint16_t, 1>(x, y, pos, rows, len, d, l2b, stream);
  return vec4 ? launch_rope_t<float, 4>(x, y, pos, rows, len, d, l2b, stream)
              : launch_rope_t<float, 1>(x, y, pos, rows, len, d, l2b, stream);
}

}  // namespace ra
