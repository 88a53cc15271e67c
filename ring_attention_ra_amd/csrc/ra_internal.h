// Internal declarations of libra.so: host-side error reporting and the kernel
// launchers each .hip file provides, plus small device helpers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra.h"

namespace ra {

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Record a formatted message as this thread's last error and return `st`.
ra_status fail(ra_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Map the result of a launch to RA_OK / RA_ERR_HIP (with the runtime's text).
ra_status launch_result(hipError_t err, const char* what);

struct PermuteArgs {
  const void* src;
  void* dst;
  int32_t* pos;
  int64_t outer;
  int64_t seq_len;
  int64_t chunk;     // C = seq_len / n_ranks
  int64_t row_bytes;
  int32_t n_ranks;
  int32_t layout;
  int32_t rank;      // -1 = all ranks
  int32_t inverse;
};

struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const float* slopes;  // [Hq] or nullptr
  float* o_acc;
  float* m;
  float* l;
  int32_t batch, heads_q, heads_kv, head_dim, len_q, len_kv;
  int32_t causal;
  float scale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const float* slopes;
  const void* d_o;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int32_t batch, heads_q, heads_kv, head_dim, len_q, len_kv;
  int32_t causal;
  float scale;
};

// One tensor (or position list) for the optional device-side checks.
enum CheckKind {
  kCheckFinite = 0,         // every element finite
  kCheckNoNanNoPosInf = 1,  // no NaN and no +Inf (-Inf allowed: m and lse of rows with no key)
  kCheckFiniteNonNeg = 2,   // finite and not negative (the running sum l)
  kCheckPositions = 3       // int32 positions: non-negative and strictly increasing
};
struct CheckItem {
  const char* name;
  const void* ptr;
  int64_t n;      // elements
  int32_t dtype;  // ra_dtype of the elements (unused for kCheckPositions)
  int32_t kind;   // CheckKind
};

// counters[i] = number of elements of items[i] that break its rule, for
// i < n_items (<= kMaxCheckItems); counters is device memory of n_items
// words, cleared here by a kernel. Enqueued on `stream`.
constexpr int kMaxCheckItems = 8;
hipError_t launch_check_counts(const CheckItem* items, int n_items, unsigned long long* counters,
                               hipStream_t stream);
// Device address of the library's static scratch counters (kMaxCheckItems
// words) on the current device; no allocation.
hipError_t scratch_counters(unsigned long long** out);

hipError_t launch_positions(int64_t seq_len, int32_t n_ranks, int32_t rank, int32_t layout,
                            int32_t* pos, hipStream_t stream);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);
hipError_t launch_state_init(float* o_acc, float* m, float* l, int64_t rows, int32_t head_dim,
                             hipStream_t stream);
hipError_t launch_fwd_fp32(const StepArgs& a, hipStream_t stream);
hipError_t launch_fwd_bf16(const StepArgs& a, hipStream_t stream);
hipError_t launch_finalize(const float* o_acc, const float* m, const float* l, void* o,
                           float* lse, int64_t rows, int32_t head_dim, int32_t dtype,
                           hipStream_t stream);
hipError_t launch_bwd_delta(const void* o, const void* d_o, float* delta, int64_t rows,
                            int32_t head_dim, int32_t dtype, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_fp32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t outer, int64_t len, int32_t d,
                       int32_t dtype, float base, hipStream_t stream);

}  // namespace ra

// ---------------------------------------------------------------------------
// device helpers (gfx950)
// ---------------------------------------------------------------------------

typedef __attribute__((ext_vector_type(8))) __bf16 ra_bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 ra_bf16x2;
typedef __attribute__((ext_vector_type(2))) float ra_f32x2;
typedef __attribute__((ext_vector_type(4))) float ra_f32x4;
typedef __attribute__((ext_vector_type(16))) float ra_f32x16;

#define RA_LOG2E 1.4426950408889634f
#define RA_LN2 0.6931471805599453f

// C[32x32] += A[32x16] * B[16x32], bf16 in, fp32 accumulate.
// Operand slots: lane l supplies row (A) / column (B) l % 32 and eight k
// values; slot i of a lane in half h = l / 32 is the same k for A and B, which
// is all the kernels rely on. Result: lane l, element e holds
// C[8*(e/4) + 4*(l/32) + e%4][l % 32].
__device__ __forceinline__ ra_f32x16 ra_mfma32(const uint4& a, const uint4& b, ra_f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(ra_bf16x8, a),
                                                 __builtin_bit_cast(ra_bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> two bf16 (round to nearest even), packed in one dword.
__device__ __forceinline__ uint32_t ra_pack_bf16(float lo, float hi) {
  ra_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, ra_bf16x2));
}

__device__ __forceinline__ float ra_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float ra_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value of x held by the partner lane in the other half of the wave
// (lane l <-> l ^ 32), via v_permlane32_swap. Of the two swap results one is
// the lane's own value and the other the partner's; picking "the one that is
// not our own bits" does not depend on which result register is which.
__device__ __forceinline__ float ra_swap_halves(float x) {
  const uint32_t own = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(own, own, false, false);
  return __uint_as_float(r[0] == own ? r[1] : r[0]);
}
