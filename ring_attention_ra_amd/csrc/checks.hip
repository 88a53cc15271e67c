// Device-side checks behind the library's optional validation: counting
// non-finite elements of a tensor (the synchronising finite check that the
// RA_CHECK_FINITE=1 switch adds to the compute entry points, and
// ra_count_nonfinite) and testing that a position list is non-negative and
// strictly increasing (the RA_DEBUG=1 switch).
//
// The finite check exists because a ring hands every chunk from device to
// device, and a corrupted transfer shows up as NaN or Inf in what a rank
// receives (discosf.com article, §5.2 典型问题排查, NaN loss and ring transfer
// corruption). These checks are HBM-bound reductions; they are not on the hot
// path and run only when asked for.
#include <mutex>
#include <vector>

#include "ra_internal.h"

namespace ra {

// Scratch of ra_count_nonfinite_noalloc: kMaxCheckItems 64-bit counters in a
// file-scope device array (64 bytes), for callers that cannot allocate. Each
// GPU the library runs on holds its own copy at its own address until the
// process ends, and every call on that GPU shares it: the counters are
// cleared at the start of each use, and calls that overlap on one GPU race.
static __device__ __align__(256) unsigned long long scratch[kMaxCheckItems];

namespace {

// True when an element breaks the rule of its check kind, from its raw bits.
template <typename U>
__device__ __forceinline__ bool bad_bits(U bits, int kind);

template <>
__device__ __forceinline__ bool bad_bits<uint16_t>(uint16_t bits, int kind) {
  const bool all_ones = (bits & 0x7f80u) == 0x7f80u;  // bf16: Inf or NaN
  if (kind == kCheckFinite) return all_ones;
  if (kind == kCheckNoNanNoPosInf) return all_ones && bits != 0xff80u;  // -Inf allowed
  return all_ones || ((bits & 0x8000u) && (bits & 0x7fffu));            // finite and >= 0
}

template <>
__device__ __forceinline__ bool bad_bits<uint32_t>(uint32_t bits, int kind) {
  const bool all_ones = (bits & 0x7f800000u) == 0x7f800000u;  // fp32: Inf or NaN
  if (kind == kCheckFinite) return all_ones;
  if (kind == kCheckNoNanNoPosInf) return all_ones && bits != 0xff800000u;
  return all_ones || ((bits & 0x80000000u) && (bits & 0x7fffffffu));
}

// counter[slot] += number of elements of x that break the rule.
template <typename U>
__global__ void count_bad_kernel(const U* __restrict__ x, int64_t n, int kind,
                                 unsigned long long* __restrict__ counter) {
  unsigned long long bad = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride)
    bad += bad_bits<U>(x[i], kind) ? 1u : 0u;
  if (bad) atomicAdd(counter, bad);
}

// counter += number of i with pos[i] < 0, or pos[i + 1] <= pos[i].
__global__ void positions_order_kernel(const int32_t* __restrict__ pos, int64_t n,
                                       unsigned long long* __restrict__ counter) {
  unsigned long long bad = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    const int32_t p = pos[i];
    bad += (p < 0 || (i + 1 < n && pos[i + 1] <= p)) ? 1u : 0u;
  }
  if (bad) atomicAdd(counter, bad);
}

// counter[0 .. n) = 0 (a kernel rather than a memset, so that the sequence can
// also run inside a captured graph).
__global__ void zero_kernel(unsigned long long* __restrict__ counter, int n) {
  if ((int)threadIdx.x < n) counter[threadIdx.x] = 0;
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 2048) b = 2048;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

// Device address of `scratch` on the current device. In host code the array's
// name is only a stand-in: the address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and is kept per device.
hipError_t scratch_counters(unsigned long long** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<unsigned long long*> per_device;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)per_device.size() <= dev) per_device.resize(dev + 1, nullptr);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = static_cast<unsigned long long*>(p);
  }
  *out = per_device[dev];
  return hipSuccess;
}

hipError_t launch_check_counts(const CheckItem* items, int n_items, unsigned long long* counters,
                               hipStream_t stream) {
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, stream, counters, n_items);
  hipError_t e = hipGetLastError();
  for (int i = 0; i < n_items && e == hipSuccess; ++i) {
    const CheckItem& it = items[i];
    if (it.n <= 0 || !it.ptr) continue;
    const dim3 grid(grid_for(it.n)), block(256);
    if (it.kind == kCheckPositions)
      hipLaunchKernelGGL(positions_order_kernel, grid, block, 0, stream,
                         static_cast<const int32_t*>(it.ptr), it.n, counters + i);
    else if (it.dtype == RA_BF16)
      hipLaunchKernelGGL(count_bad_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(it.ptr), it.n, it.kind, counters + i);
    else
      hipLaunchKernelGGL(count_bad_kernel<uint32_t>, grid, block, 0, stream,
                         static_cast<const uint32_t*>(it.ptr), it.n, it.kind, counters + i);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ra
