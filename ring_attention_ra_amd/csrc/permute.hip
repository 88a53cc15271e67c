// Position index and layout permutation kernels.
//
// Contiguous split: rank r holds tokens [r*C, (r+1)*C) (discosf.com article,
// §2.1 序列切分策略对比). Zig-zag: token i goes to rank i mod N, so rank r holds
// r, r+N, r+2N, ... (digipub.cc "大模型如何訓練百萬 Token 上下文", section
// "Zig Zag Ring Attention"). Local row t of rank r is global row pos_r(t).
//
// The permutation is pure data movement: every output row is one input row,
// copied in the widest aligned unit (16, 8, 4 or 2 bytes) by consecutive
// lanes, so a 256-byte row is read and written by 16 adjacent lanes.
#include "ra_internal.h"

namespace ra {
namespace {

__device__ __forceinline__ int64_t pos_of(int64_t r, int64_t t, int64_t C, int64_t N, int layout) {
  return layout == RA_CONTIGUOUS ? r * C + t : t * N + r;
}

__global__ void positions_kernel(int32_t* __restrict__ pos, int64_t total, int64_t C, int64_t N,
                                 int32_t rank, int layout) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = rank < 0 ? i / C : rank;
    const int64_t t = rank < 0 ? i - (i / C) * C : i;
    pos[i] = (int32_t)pos_of(r, t, C, N, layout);
  }
}

// One thread per copy unit of type T. `units` copy units per row.
// Output rows are enumerated in output order; each maps to one input row.
template <typename T>
__global__ void permute_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t out_rows,
                               uint32_t units, int64_t outer, int64_t S, int64_t C, int64_t N,
                               int32_t rank, int layout, int inverse) {
  const int64_t total = out_rows * units;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / units;
    const int64_t u = i - row * units;
    int64_t in_row, out_row = row;
    if (!inverse) {
      // out: [N?, outer, C] (rank-major) <- in: [outer, S] (global)
      const int64_t per_rank = outer * C;
      const int64_t r = rank < 0 ? row / per_rank : rank;
      const int64_t rem = rank < 0 ? row - r * per_rank : row;
      const int64_t o = rem / C;
      const int64_t t = rem - o * C;
      in_row = o * S + pos_of(r, t, C, N, layout);
    } else if (rank < 0) {
      // out: [outer, S] (global) <- in: [N, outer, C]
      const int64_t o = row / S;
      const int64_t p = row - o * S;
      const int64_t r = layout == RA_CONTIGUOUS ? p / C : p % N;
      const int64_t t = layout == RA_CONTIGUOUS ? p - r * C : p / N;
      in_row = (r * outer + o) * C + t;
    } else {
      // out: the rows of one rank inside [outer, S] <- in: [outer, C]
      const int64_t o = row / C;
      const int64_t t = row - o * C;
      in_row = row;
      out_row = o * S + pos_of(rank, t, C, N, layout);
    }
    dst[out_row * units + u] = src[in_row * units + u];
  }
}

unsigned grid_for(int64_t work, int threads) {
  int64_t blocks = (work + threads - 1) / threads;
  const int64_t cap = 256 * 64;  // grid-stride beyond this
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

template <typename T>
hipError_t launch_typed(const PermuteArgs& a, int64_t out_rows, hipStream_t stream) {
  const uint32_t units = (uint32_t)(a.row_bytes / (int64_t)sizeof(T));
  const int threads = 256;
  hipLaunchKernelGGL(permute_kernel<T>, dim3(grid_for(out_rows * units, threads)), dim3(threads),
                     0, stream, (const T*)a.src, (T*)a.dst, out_rows, units, a.outer, a.seq_len,
                     a.chunk, (int64_t)a.n_ranks, a.rank, a.layout, a.inverse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_positions(int64_t seq_len, int32_t n_ranks, int32_t rank, int32_t layout,
                            int32_t* pos, hipStream_t stream) {
  const int64_t C = seq_len / n_ranks;
  const int64_t total = rank < 0 ? seq_len : C;
  hipLaunchKernelGGL(positions_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, pos,
                     total, C, (int64_t)n_ranks, rank, layout);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  int64_t out_rows;
  if (!a.inverse)
    out_rows = a.outer * a.chunk * (a.rank < 0 ? a.n_ranks : 1);
  else
    out_rows = a.rank < 0 ? a.outer * a.seq_len : a.outer * a.chunk;
  const uintptr_t align = (uintptr_t)a.src | (uintptr_t)a.dst | (uintptr_t)a.row_bytes;
  if (align % 16 == 0) return launch_typed<uint4>(a, out_rows, stream);
  if (align % 8 == 0) return launch_typed<uint2>(a, out_rows, stream);
  if (align % 4 == 0) return launch_typed<uint32_t>(a, out_rows, stream);
  return launch_typed<uint16_t>(a, out_rows, stream);
}

}  // namespace ra
