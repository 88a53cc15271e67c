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
#include <algorithm>

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
// Index arithmetic in I: 32-bit unsigned when every row index times the units
// per row fits (the common case; 64-bit division costs dozens of
// instructions per element), 64-bit otherwise.
template <typename T, typename I>
__global__ void permute_kernel(const T* __restrict__ src, T* __restrict__ dst, I out_rows, I units, I outer,
                               I S, I C, I N, int32_t rank, int layout, int inverse) {
  const I total = out_rows * units;
  for (I i = blockIdx.x * (I)blockDim.x + threadIdx.x; i < total; i += (I)gridDim.x * blockDim.x) {
    const I row = i / units;
    const I u = i - row * units;
    I in_row, out_row = row;
    if (!inverse) {
      // out: [N?, outer, C] (rank-major) <- in: [outer, S] (global)
      const I per_rank = outer * C;
      const I r = rank < 0 ? row / per_rank : (I)rank;
      const I rem = rank < 0 ? row - r * per_rank : row;
      const I o = rem / C;
      const I t = rem - o * C;
      in_row = o * S + (layout == RA_CONTIGUOUS ? r * C + t : t * N + r);
    } else if (rank < 0) {
      // out: [outer, S] (global) <- in: [N, outer, C]
      const I o = row / S;
      const I p = row - o * S;
      const I r = layout == RA_CONTIGUOUS ? p / C : p % N;
      const I t = layout == RA_CONTIGUOUS ? p - r * C : p / N;
      in_row = (r * outer + o) * C + t;
    } else {
      // out: the rows of one rank inside [outer, S] <- in: [outer, C]
      const I o = row / C;
      const I t = row - o * C;
      in_row = row;
      out_row = o * S + (layout == RA_CONTIGUOUS ? (I)rank * C + t : t * N + (I)rank);
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
  const int64_t units = a.row_bytes / (int64_t)sizeof(T);
  const int threads = 256;
  const dim3 grid(grid_for(out_rows * units, threads));
  // Largest row index either side can hold: the global [outer, S] tensor or
  // the rank-major one; 32-bit indices if every element index fits.
  const int64_t rows_max = std::max(a.outer * a.seq_len, out_rows);
  if ((rows_max + 1) * units < ((int64_t)1 << 32) - (int64_t)grid.x * threads)
    hipLaunchKernelGGL((permute_kernel<T, uint32_t>), grid, dim3(threads), 0, stream, (const T*)a.src, (T*)a.dst,
                       (uint32_t)out_rows, (uint32_t)units, (uint32_t)a.outer, (uint32_t)a.seq_len,
                       (uint32_t)a.chunk, (uint32_t)a.n_ranks, a.rank, a.layout, a.inverse);
  else
    hipLaunchKernelGGL((permute_kernel<T, int64_t>), grid, dim3(threads), 0, stream, (const T*)a.src, (T*)a.dst,
                       out_rows, units, a.outer, a.seq_len, a.chunk, (int64_t)a.n_ranks, a.rank, a.layout,
                       a.inverse);
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
