// C entry points of libra.so: argument validation on the host, then dispatch
// to the kernels. Nothing is launched unless every argument is valid.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <cstring>

#include "ra_internal.h"

namespace ra {

static thread_local char g_err[512] = "";

ra_status fail(ra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ra_status launch_result(hipError_t err, const char* what) {
  if (err == hipSuccess) return RA_OK;
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool dtype_ok(int32_t dt) { return dt == RA_BF16 || dt == RA_FP32; }
static int64_t dtype_size(int32_t dt) { return dt == RA_BF16 ? 2 : 4; }

static ra_status check_seq(int64_t seq_len, int32_t n_ranks, int32_t layout, int32_t rank) {
  if (n_ranks <= 0) return fail(RA_ERR_INVALID_ARGUMENT, "n_ranks must be positive (got %d)", n_ranks);
  if (seq_len <= 0 || seq_len % n_ranks)
    return fail(RA_ERR_INVALID_ARGUMENT, "seq_len %lld must be a positive multiple of n_ranks %d",
                (long long)seq_len, n_ranks);
  if (seq_len > INT32_MAX)
    return fail(RA_ERR_INVALID_ARGUMENT, "seq_len %lld exceeds the int32 position range",
                (long long)seq_len);
  if (layout != RA_CONTIGUOUS && layout != RA_ZIGZAG)
    return fail(RA_ERR_INVALID_ARGUMENT, "unknown layout %d", layout);
  if (rank < -1 || rank >= n_ranks)
    return fail(RA_ERR_INVALID_ARGUMENT, "rank %d out of range [-1, %d)", rank, n_ranks);
  return RA_OK;
}

// Shared checks of the per-step entry points. Sets *empty when there is no
// work (a zero dimension).
static ra_status check_dims(const ra_dims* d, bool* empty) {
  if (!d) return fail(RA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->batch < 0 || d->heads_q < 0 || d->heads_kv < 0 || d->len_q < 0 || d->len_kv < 0)
    return fail(RA_ERR_INVALID_ARGUMENT, "negative dimension");
  if (!dtype_ok(d->dtype)) return fail(RA_ERR_INVALID_ARGUMENT, "unknown dtype %d", d->dtype);
  if (d->head_dim <= 0) return fail(RA_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  if (d->heads_q > 0 && (d->heads_kv <= 0 || d->heads_q % d->heads_kv))
    return fail(RA_ERR_INVALID_ARGUMENT, "heads_q %d must be a positive multiple of heads_kv %d",
                d->heads_q, d->heads_kv);
  if (d->dtype == RA_BF16 && d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "bf16 head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->dtype == RA_FP32 && d->head_dim > 128)
    return fail(RA_ERR_UNSUPPORTED, "fp32 head_dim must be at most 128 (got %d)", d->head_dim);
  *empty = d->batch == 0 || d->heads_q == 0 || d->len_q == 0;
  return RA_OK;
}

}  // namespace ra

using namespace ra;

extern "C" {

int32_t ra_abi_version(void) { return 1; }

const char* ra_last_error(void) { return g_err; }

ra_status ra_positions(int64_t seq_len, int32_t n_ranks, int32_t rank, int32_t layout,
                       int32_t* pos_out, void* stream) {
  ra_status st = check_seq(seq_len, n_ranks, layout, rank);
  if (st != RA_OK) return st;
  if (!pos_out) return fail(RA_ERR_INVALID_ARGUMENT, "pos_out is NULL");
  return launch_result(
      launch_positions(seq_len, n_ranks, rank, layout, pos_out, (hipStream_t)stream),
      "ra_positions");
}

ra_status ra_layout_permute(const void* src, void* dst, int32_t* pos, int64_t outer,
                            int64_t seq_len, int32_t row_elems, int32_t dtype, int32_t n_ranks,
                            int32_t layout, int32_t rank, int32_t inverse, void* stream) {
  ra_status st = check_seq(seq_len, n_ranks, layout, rank);
  if (st != RA_OK) return st;
  if (outer < 0) return fail(RA_ERR_INVALID_ARGUMENT, "outer must be non-negative");
  if (row_elems <= 0) return fail(RA_ERR_INVALID_ARGUMENT, "row_elems must be positive");
  if (!dtype_ok(dtype)) return fail(RA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (inverse != 0 && inverse != 1)
    return fail(RA_ERR_INVALID_ARGUMENT, "inverse must be 0 or 1");
  const int64_t row_bytes = (int64_t)row_elems * dtype_size(dtype);
  const int64_t chunk = seq_len / n_ranks;
  const int64_t global_bytes = outer * seq_len * row_bytes;
  const int64_t ranked_bytes = outer * chunk * row_bytes * (rank < 0 ? n_ranks : 1);
  if (outer > 0) {
    if (!src || !dst) return fail(RA_ERR_INVALID_ARGUMENT, "src or dst is NULL");
    const char* s = (const char*)src;
    const char* e = (const char*)dst;
    const int64_t sb = inverse ? ranked_bytes : global_bytes;
    const int64_t db = inverse ? global_bytes : ranked_bytes;
    if (s < e + db && e < s + sb) return fail(RA_ERR_INVALID_ARGUMENT, "src and dst overlap");
  }
  if (pos) {
    st = launch_result(launch_positions(seq_len, n_ranks, rank, layout, pos, (hipStream_t)stream),
                       "ra_layout_permute(positions)");
    if (st != RA_OK) return st;
  }
  if (outer == 0) return RA_OK;
  PermuteArgs a{src, dst, pos, outer, seq_len, chunk, row_bytes, n_ranks, layout, rank, inverse};
  return launch_result(launch_permute(a, (hipStream_t)stream), "ra_layout_permute");
}

ra_status ra_rope(const void* x, void* y, const int32_t* pos, int64_t outer, int64_t len,
                  int32_t head_dim, int32_t dtype, float base, void* stream) {
  if (outer < 0 || len < 0) return fail(RA_ERR_INVALID_ARGUMENT, "negative outer or len");
  if (!dtype_ok(dtype)) return fail(RA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (head_dim < 2 || head_dim > 256 || head_dim % 2)
    return fail(RA_ERR_INVALID_ARGUMENT, "head_dim must be even and in [2, 256] (got %d)", head_dim);
  if (!(base > 0.0f) || !std::isfinite(base))
    return fail(RA_ERR_INVALID_ARGUMENT, "base must be positive and finite");
  if (outer == 0 || len == 0) return RA_OK;
  if (!x || !y || !pos) return fail(RA_ERR_INVALID_ARGUMENT, "x, y or pos is NULL");
  const int64_t bytes = outer * len * head_dim * dtype_size(dtype);
  const char* xs = (const char*)x;
  const char* ys = (const char*)y;
  if (xs != ys && xs < ys + bytes && ys < xs + bytes)
    return fail(RA_ERR_INVALID_ARGUMENT, "x and y overlap without being the same tensor");
  return launch_result(launch_rope(x, y, pos, outer, len, head_dim, dtype, base, (hipStream_t)stream),
                       "ra_rope");
}

ra_status ra_state_init(const ra_dims* d, float* o_acc, float* m, float* l, void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (empty) return RA_OK;
  if (!o_acc || !m || !l) return fail(RA_ERR_INVALID_ARGUMENT, "o_acc, m or l is NULL");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  return launch_result(launch_state_init(o_acc, m, l, rows, d->head_dim, (hipStream_t)stream),
                       "ra_state_init");
}

ra_status ra_step_fwd(const ra_dims* d, const void* q, const void* k_blk, const void* v_blk,
                      const int32_t* q_pos, const int32_t* k_pos, int32_t causal, float scale,
                      const float* alibi_slopes, float* o_acc, float* m, float* l, void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (!std::isfinite(scale)) return fail(RA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (empty || d->len_kv == 0) return RA_OK;
  if (!q || !k_blk || !v_blk || !q_pos || !k_pos || !o_acc || !m || !l)
    return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (d->dtype == RA_BF16 && !(aligned16(q) && aligned16(k_blk) && aligned16(v_blk) && aligned16(o_acc)))
    return fail(RA_ERR_INVALID_ARGUMENT, "bf16 q, k_blk, v_blk and o_acc must be 16-byte aligned");
  StepArgs a{q, k_blk, v_blk, q_pos, k_pos, alibi_slopes, o_acc, m, l,
             d->batch, d->heads_q, d->heads_kv, d->head_dim, d->len_q, d->len_kv,
             causal ? 1 : 0, scale};
  if (d->dtype == RA_BF16)
    return launch_result(launch_fwd_bf16(a, (hipStream_t)stream), "ra_step_fwd(bf16)");
  return launch_result(launch_fwd_fp32(a, (hipStream_t)stream), "ra_step_fwd(fp32)");
}

ra_status ra_finalize(const ra_dims* d, const float* o_acc, const float* m, const float* l,
                      void* o, float* lse, void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (empty || (!o && !lse)) return RA_OK;
  if (!m || !l || (o && !o_acc)) return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  return launch_result(
      launch_finalize(o_acc, m, l, o, lse, rows, d->head_dim, d->dtype, (hipStream_t)stream),
      "ra_finalize");
}

ra_status ra_bwd_delta(const ra_dims* d, const void* o, const void* d_o, float* delta,
                       void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (empty) return RA_OK;
  if (!o || !d_o || !delta) return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  return launch_result(
      launch_bwd_delta(o, d_o, delta, rows, d->head_dim, d->dtype, (hipStream_t)stream),
      "ra_bwd_delta");
}

ra_status ra_step_bwd(const ra_dims* d, const void* q, const void* k_blk, const void* v_blk,
                      const int32_t* q_pos, const int32_t* k_pos, int32_t causal, float scale,
                      const float* alibi_slopes, const void* d_o, const float* lse,
                      const float* delta, float* dq_acc, float* dk_blk, float* dv_blk,
                      void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (!std::isfinite(scale)) return fail(RA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (d->dtype != RA_BF16 || d->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "ra_step_bwd supports bf16 with head_dim 128 only");
  if (empty || d->len_kv == 0 || d->batch == 0) return RA_OK;
  if (!q || !k_blk || !v_blk || !q_pos || !k_pos || !d_o || !lse || !delta || !dq_acc ||
      !dk_blk || !dv_blk)
    return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!(aligned16(q) && aligned16(k_blk) && aligned16(v_blk) && aligned16(d_o) && aligned16(dq_acc) &&
        aligned16(dk_blk) && aligned16(dv_blk)))
    return fail(RA_ERR_INVALID_ARGUMENT, "ra_step_bwd tensors must be 16-byte aligned");
  BwdArgs a{q, k_blk, v_blk, q_pos, k_pos, alibi_slopes, d_o, lse, delta, dq_acc, dk_blk, dv_blk,
            d->batch, d->heads_q, d->heads_kv, d->head_dim, d->len_q, d->len_kv,
            causal ? 1 : 0, scale};
  return launch_result(launch_bwd_bf16(a, (hipStream_t)stream), "ra_step_bwd");
}

}  // extern "C"
