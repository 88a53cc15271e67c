// Row-wise kernels around the attention step: accumulator start state, the
// final normalisation o = o_acc / l, lse = m + ln l (intelliparadigm.com
// long-context survey, §3.1.2 FlashAttention的核心算法: the running max starts
// at -inf, the running sum at 0, and the output is divided by l at the end),
// and the backward row term delta = <d_o, o>.
#include "ra_internal.h"

namespace ra {
namespace {

unsigned blocks_for(int64_t work, int threads) {
  int64_t b = (work + threads - 1) / threads;
  if (b > 256 * 64) b = 256 * 64;
  return (unsigned)(b < 1 ? 1 : b);
}

__global__ void state_init_kernel(float* __restrict__ o_acc, float* __restrict__ m,
                                  float* __restrict__ l, int64_t rows, int32_t head_dim) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t first = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t n = rows * head_dim;
  for (int64_t i = first; i < n; i += stride) o_acc[i] = 0.0f;
  for (int64_t i = first; i < rows; i += stride) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
  }
}

// One thread per 4 consecutive elements of a row (head_dim % 4 == 0), or per
// element otherwise.
template <int VEC, bool BF16>
__global__ void finalize_kernel(const float* __restrict__ o_acc, const float* __restrict__ m,
                                const float* __restrict__ l, void* __restrict__ o,
                                float* __restrict__ lse, int64_t rows, int32_t head_dim) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t first = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (o) {
    const int32_t per_row = head_dim / VEC;
    const int64_t n = rows * per_row;
    for (int64_t i = first; i < n; i += stride) {
      const int64_t row = i / per_row;
      const float lv = l[row];
      const float inv = lv > 0.0f ? 1.0f / lv : 0.0f;
      if constexpr (VEC == 4) {
        const float4 a = reinterpret_cast<const float4*>(o_acc)[i];
        if constexpr (BF16) {
          uint2 w;
          w.x = ra_pack_bf16(a.x * inv, a.y * inv);
          w.y = ra_pack_bf16(a.z * inv, a.w * inv);
          reinterpret_cast<uint2*>(o)[i] = w;
        } else {
          reinterpret_cast<float4*>(o)[i] = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
        }
      } else {
        const float v = o_acc[i] * inv;
        if constexpr (BF16) {
          const uint32_t w = ra_pack_bf16(v, 0.0f);
          reinterpret_cast<uint16_t*>(o)[i] = (uint16_t)(w & 0xffffu);
        } else {
          reinterpret_cast<float*>(o)[i] = v;
        }
      }
    }
  }
  if (lse) {
    for (int64_t i = first; i < rows; i += stride) {
      const float lv = l[i];
      lse[i] = lv > 0.0f ? m[i] + logf(lv) : -INFINITY;
    }
  }
}

// 16 lanes per row; each lane reads head_dim/16 elements of o and d_o.
template <bool BF16>
__global__ void bwd_delta_kernel(const void* __restrict__ o, const void* __restrict__ d_o,
                                 float* __restrict__ delta, int64_t rows, int32_t head_dim) {
  const int64_t groups = (int64_t)gridDim.x * (blockDim.x / 16);
  const int sub = threadIdx.x & 15;
  for (int64_t row = blockIdx.x * (int64_t)(blockDim.x / 16) + threadIdx.x / 16; row < rows;
       row += groups) {
    float acc = 0.0f;
    for (int d = sub; d < head_dim; d += 16) {
      const int64_t idx = row * head_dim + d;
      float a, b;
      if constexpr (BF16) {
        a = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(o)[idx] << 16);
        b = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(d_o)[idx] << 16);
      } else {
        a = reinterpret_cast<const float*>(o)[idx];
        b = reinterpret_cast<const float*>(d_o)[idx];
      }
      acc = fmaf(a, b, acc);
    }
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (sub == 0) delta[row] = acc;
  }
}

}  // namespace

hipError_t launch_state_init(float* o_acc, float* m, float* l, int64_t rows, int32_t head_dim,
                             hipStream_t stream) {
  hipLaunchKernelGGL(state_init_kernel, dim3(blocks_for(rows * head_dim, 256)), dim3(256), 0,
                     stream, o_acc, m, l, rows, head_dim);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* o_acc, const float* m, const float* l, void* o, float* lse,
                           int64_t rows, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const bool vec4 = head_dim % 4 == 0 && ((uintptr_t)o_acc & 15u) == 0 &&
                    ((uintptr_t)o & (dtype == RA_BF16 ? 7u : 15u)) == 0;
  const int64_t work = o ? rows * (vec4 ? head_dim / 4 : head_dim) : rows;
  const dim3 grid(blocks_for(work, 256)), block(256);
  if (dtype == RA_BF16) {
    if (vec4)
      hipLaunchKernelGGL((finalize_kernel<4, true>), grid, block, 0, stream, o_acc, m, l, o, lse,
                         rows, head_dim);
    else
      hipLaunchKernelGGL((finalize_kernel<1, true>), grid, block, 0, stream, o_acc, m, l, o, lse,
                         rows, head_dim);
  } else {
    if (vec4)
      hipLaunchKernelGGL((finalize_kernel<4, false>), grid, block, 0, stream, o_acc, m, l, o, lse,
                         rows, head_dim);
    else
      hipLaunchKernelGGL((finalize_kernel<1, false>), grid, block, 0, stream, o_acc, m, l, o, lse,
                         rows, head_dim);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const void* o, const void* d_o, float* delta, int64_t rows,
                            int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const dim3 grid(blocks_for(rows * 16, 256)), block(256);
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(bwd_delta_kernel<true>, grid, block, 0, stream, o, d_o, delta, rows,
                       head_dim);
  else
    hipLaunchKernelGGL(bwd_delta_kernel<false>, grid, block, 0, stream, o, d_o, delta, rows,
                       head_dim);
  return hipGetLastError();
}

}  // namespace ra
