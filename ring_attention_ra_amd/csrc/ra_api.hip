// C entry points of libra.so: argument validation on the host, then dispatch
// to the kernels. Nothing is launched unless every argument is valid.
#include <stdarg.h>
#include <stdio.h>

#include <stdlib.h>

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

// Limits of the bf16 matrix-core kernels. They address one head's slab of a
// tensor through a buffer resource, whose byte count is a signed 32-bit value,
// and index rows as int32 row * head_dim; the fp32 state slab of a head
// (len_q * head_dim * 4 bytes) is the widest such slab. The grid has one
// work-group per 128 or 256 rows of each head.
constexpr int64_t kSlabLimit = (int64_t)1 << 31;

static ra_status check_bf16_limits(const ra_dims* d, bool backward) {
  const int64_t q_slab = (int64_t)d->len_q * d->head_dim * (backward ? 2 : 4);
  const int64_t kv_slab = (int64_t)d->len_kv * d->head_dim * 2;
  if (q_slab >= kSlabLimit)
    return fail(RA_ERR_UNSUPPORTED,
                "len_q %d x head_dim %d: one head's %s slab would be %lld bytes, beyond the 2^31 - 1 "
                "that the bf16 kernels address", d->len_q, d->head_dim, backward ? "q / d_o" : "o_acc",
                (long long)q_slab);
  if (backward && kv_slab >= kSlabLimit)
    return fail(RA_ERR_UNSUPPORTED,
                "len_kv %d x head_dim %d: one head's k / v slab would be %lld bytes, beyond the 2^31 - 1 "
                "that the bf16 kernels address", d->len_kv, d->head_dim, (long long)kv_slab);
  const int64_t tiles_q = ((int64_t)d->len_q + 127) / 128;
  const int64_t tiles_k = ((int64_t)d->len_kv + 127) / 128;
  if (tiles_q * d->batch * d->heads_q > INT32_MAX || tiles_k * d->batch * d->heads_kv > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "batch x heads x row tiles exceeds the int32 grid");
  return RA_OK;
}

static ra_status check_fp32_limits(const ra_dims* d) {
  // one work-group per 32 rows of a head at most
  if (((int64_t)d->len_q + 31) / 32 * d->batch * d->heads_q > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "batch x heads x row tiles exceeds the int32 grid");
  return RA_OK;
}

// The optional checks are switched on per process by environment variables,
// read at every call: RA_CHECK_FINITE=1 (finite inputs and outputs) and
// RA_DEBUG=1 (position order).
static bool env_on(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && strcmp(v, "0") != 0;
}

// Runs the checks of items[0 .. n) on `stream` with the device counters
// `dev`, waits for them, and returns RA_OK or `bad_status` naming the first
// item that failed (or, with counts_out, the counts of every item).
static ra_status run_checks_with(unsigned long long* dev, const CheckItem* items, int n, hipStream_t stream,
                                 const char* entry, const char* when, ra_status bad_status,
                                 int64_t* counts_out) {
  unsigned long long host[kMaxCheckItems] = {};
  hipError_t e = launch_check_counts(items, n, dev, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(host, dev, n * sizeof(unsigned long long), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return launch_result(e, "device check");
  for (int i = 0; i < n; ++i) {
    if (counts_out) counts_out[i] = (int64_t)host[i];
    if (host[i] == 0 || counts_out) continue;
    if (items[i].kind == kCheckPositions)
      return fail(bad_status, "%s: %s is not non-negative and strictly increasing (%llu bad entries)",
                  entry, items[i].name, host[i]);
    return fail(bad_status, "%s: %s holds %llu %s value(s) %s", entry, items[i].name, host[i],
                items[i].kind == kCheckFinite ? "non-finite"
                : items[i].kind == kCheckNoNanNoPosInf ? "NaN or +Inf" : "non-finite or negative",
                when);
  }
  return RA_OK;
}

// The same with a device counter array allocated for the call.
static ra_status run_checks(const CheckItem* items, int n, hipStream_t stream, const char* entry,
                            const char* when, ra_status bad_status, int64_t* counts_out = nullptr) {
  unsigned long long* dev = nullptr;
  hipError_t e = hipMalloc(&dev, kMaxCheckItems * sizeof(unsigned long long));
  if (e != hipSuccess) return launch_result(e, "check counters");
  const ra_status st = run_checks_with(dev, items, n, stream, entry, when, bad_status, counts_out);
  e = hipFree(dev);
  if (st == RA_OK && e != hipSuccess) return launch_result(e, "check counters");
  return st;
}

static CheckItem item(const char* name, const void* p, int64_t n, int32_t dtype, int32_t kind) {
  return CheckItem{name, p, n, dtype, kind};
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
  const int64_t elems = outer * len * head_dim;
  const int64_t bytes = elems * dtype_size(dtype);
  const char* xs = (const char*)x;
  const char* ys = (const char*)y;
  if (xs != ys && xs < ys + bytes && ys < xs + bytes)
    return fail(RA_ERR_INVALID_ARGUMENT, "x and y overlap without being the same tensor");
  hipStream_t st = (hipStream_t)stream;
  const bool finite = env_on("RA_CHECK_FINITE");
  if (finite) {
    const CheckItem in[] = {item("x", x, elems, dtype, kCheckFinite)};
    ra_status r = run_checks(in, 1, st, "ra_rope", "(nothing was launched)", RA_ERR_NONFINITE);
    if (r != RA_OK) return r;
  }
  ra_status r = launch_result(launch_rope(x, y, pos, outer, len, head_dim, dtype, base, st), "ra_rope");
  if (r != RA_OK || !finite) return r;
  const CheckItem out[] = {item("y", y, elems, dtype, kCheckFinite)};
  return run_checks(out, 1, st, "ra_rope", "after the rotation", RA_ERR_NONFINITE);
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
  st = d->dtype == RA_BF16 ? check_bf16_limits(d, false) : check_fp32_limits(d);
  if (st != RA_OK) return st;
  if (!q || !k_blk || !v_blk || !q_pos || !k_pos || !o_acc || !m || !l)
    return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (d->dtype == RA_BF16 && !(aligned16(q) && aligned16(k_blk) && aligned16(v_blk) && aligned16(o_acc)))
    return fail(RA_ERR_INVALID_ARGUMENT, "bf16 q, k_blk, v_blk and o_acc must be 16-byte aligned");
  hipStream_t hs = (hipStream_t)stream;
  if (env_on("RA_DEBUG")) {
    const CheckItem pi[] = {item("q_pos", q_pos, d->len_q, 0, kCheckPositions),
                            item("k_pos", k_pos, d->len_kv, 0, kCheckPositions)};
    st = run_checks(pi, 2, hs, "ra_step_fwd", "", RA_ERR_INVALID_ARGUMENT);
    if (st != RA_OK) return st;
  }
  const bool finite = env_on("RA_CHECK_FINITE");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  const int64_t kv = (int64_t)d->batch * d->heads_kv * d->len_kv * d->head_dim;
  if (finite) {
    const CheckItem in[] = {item("q", q, rows * d->head_dim, d->dtype, kCheckFinite),
                            item("k_blk", k_blk, kv, d->dtype, kCheckFinite),
                            item("v_blk", v_blk, kv, d->dtype, kCheckFinite),
                            item("alibi_slopes", alibi_slopes, alibi_slopes ? d->heads_q : 0, RA_FP32,
                                 kCheckFinite)};
    st = run_checks(in, 4, hs, "ra_step_fwd", "(nothing was launched; the state is unchanged)",
                    RA_ERR_NONFINITE);
    if (st != RA_OK) return st;
  }
  StepArgs a{q, k_blk, v_blk, q_pos, k_pos, alibi_slopes, o_acc, m, l,
             d->batch, d->heads_q, d->heads_kv, d->head_dim, d->len_q, d->len_kv,
             causal ? 1 : 0, scale};
  st = d->dtype == RA_BF16 ? launch_result(launch_fwd_bf16(a, hs), "ra_step_fwd(bf16)")
                           : launch_result(launch_fwd_fp32(a, hs), "ra_step_fwd(fp32)");
  if (st != RA_OK || !finite) return st;
  const CheckItem out[] = {item("o_acc", o_acc, rows * d->head_dim, RA_FP32, kCheckFinite),
                           item("m", m, rows, RA_FP32, kCheckNoNanNoPosInf),
                           item("l", l, rows, RA_FP32, kCheckFiniteNonNeg)};
  return run_checks(out, 3, hs, "ra_step_fwd", "after the step", RA_ERR_NONFINITE);
}

ra_status ra_finalize(const ra_dims* d, const float* o_acc, const float* m, const float* l,
                      void* o, float* lse, void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (empty || (!o && !lse)) return RA_OK;
  if (!m || !l || (o && !o_acc)) return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  hipStream_t hs = (hipStream_t)stream;
  const bool finite = env_on("RA_CHECK_FINITE");
  if (finite) {
    const CheckItem in[] = {item("o_acc", o ? o_acc : nullptr, rows * d->head_dim, RA_FP32, kCheckFinite),
                            item("m", m, rows, RA_FP32, kCheckNoNanNoPosInf),
                            item("l", l, rows, RA_FP32, kCheckFiniteNonNeg)};
    st = run_checks(in, 3, hs, "ra_finalize", "(nothing was launched)", RA_ERR_NONFINITE);
    if (st != RA_OK) return st;
  }
  st = launch_result(launch_finalize(o_acc, m, l, o, lse, rows, d->head_dim, d->dtype, hs), "ra_finalize");
  if (st != RA_OK || !finite) return st;
  const CheckItem out[] = {item("o", o, rows * d->head_dim, d->dtype, kCheckFinite),
                           item("lse", lse, rows, RA_FP32, kCheckNoNanNoPosInf)};
  return run_checks(out, 2, hs, "ra_finalize", "after the normalisation", RA_ERR_NONFINITE);
}

ra_status ra_bwd_delta(const ra_dims* d, const void* o, const void* d_o, float* delta,
                       void* stream) {
  bool empty = false;
  ra_status st = check_dims(d, &empty);
  if (st != RA_OK) return st;
  if (empty) return RA_OK;
  if (!o || !d_o || !delta) return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  hipStream_t hs = (hipStream_t)stream;
  const bool finite = env_on("RA_CHECK_FINITE");
  if (finite) {
    const CheckItem in[] = {item("o", o, rows * d->head_dim, d->dtype, kCheckFinite),
                            item("d_o", d_o, rows * d->head_dim, d->dtype, kCheckFinite)};
    st = run_checks(in, 2, hs, "ra_bwd_delta", "(nothing was launched)", RA_ERR_NONFINITE);
    if (st != RA_OK) return st;
  }
  st = launch_result(launch_bwd_delta(o, d_o, delta, rows, d->head_dim, d->dtype, hs), "ra_bwd_delta");
  if (st != RA_OK || !finite) return st;
  const CheckItem out[] = {item("delta", delta, rows, RA_FP32, kCheckFinite)};
  return run_checks(out, 1, hs, "ra_bwd_delta", "after the reduction", RA_ERR_NONFINITE);
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
  if (d->dtype == RA_BF16 && d->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "ra_step_bwd supports bf16 with head_dim 128 (got %d)", d->head_dim);
  if (empty || d->len_kv == 0 || d->batch == 0) return RA_OK;
  st = d->dtype == RA_BF16 ? check_bf16_limits(d, true) : check_fp32_limits(d);
  if (st != RA_OK) return st;
  if (!q || !k_blk || !v_blk || !q_pos || !k_pos || !d_o || !lse || !delta || !dq_acc ||
      !dk_blk || !dv_blk)
    return fail(RA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (d->dtype == RA_BF16 && !(aligned16(q) && aligned16(k_blk) && aligned16(v_blk) && aligned16(d_o) &&
                               aligned16(dq_acc) && aligned16(dk_blk) && aligned16(dv_blk)))
    return fail(RA_ERR_INVALID_ARGUMENT, "bf16 ra_step_bwd tensors must be 16-byte aligned");
  hipStream_t hs = (hipStream_t)stream;
  if (env_on("RA_DEBUG")) {
    const CheckItem pi[] = {item("q_pos", q_pos, d->len_q, 0, kCheckPositions),
                            item("k_pos", k_pos, d->len_kv, 0, kCheckPositions)};
    st = run_checks(pi, 2, hs, "ra_step_bwd", "", RA_ERR_INVALID_ARGUMENT);
    if (st != RA_OK) return st;
  }
  const bool finite = env_on("RA_CHECK_FINITE");
  const int64_t rows = (int64_t)d->batch * d->heads_q * d->len_q;
  const int64_t kv = (int64_t)d->batch * d->heads_kv * d->len_kv * d->head_dim;
  if (finite) {
    const CheckItem in[] = {item("q", q, rows * d->head_dim, d->dtype, kCheckFinite),
                            item("k_blk", k_blk, kv, d->dtype, kCheckFinite),
                            item("v_blk", v_blk, kv, d->dtype, kCheckFinite),
                            item("d_o", d_o, rows * d->head_dim, d->dtype, kCheckFinite),
                            item("lse", lse, rows, RA_FP32, kCheckNoNanNoPosInf),
                            item("delta", delta, rows, RA_FP32, kCheckFinite),
                            item("alibi_slopes", alibi_slopes, alibi_slopes ? d->heads_q : 0, RA_FP32,
                                 kCheckFinite)};
    st = run_checks(in, 7, hs, "ra_step_bwd", "(nothing was launched)", RA_ERR_NONFINITE);
    if (st != RA_OK) return st;
  }
  BwdArgs a{q, k_blk, v_blk, q_pos, k_pos, alibi_slopes, d_o, lse, delta, dq_acc, dk_blk, dv_blk,
            d->batch, d->heads_q, d->heads_kv, d->head_dim, d->len_q, d->len_kv,
            causal ? 1 : 0, scale};
  st = d->dtype == RA_BF16 ? launch_result(launch_bwd_bf16(a, hs), "ra_step_bwd(bf16)")
                           : launch_result(launch_bwd_fp32(a, hs), "ra_step_bwd(fp32)");
  if (st != RA_OK || !finite) return st;
  const CheckItem out[] = {item("dq_acc", dq_acc, rows * d->head_dim, RA_FP32, kCheckFinite),
                           item("dk_blk", dk_blk, kv, RA_FP32, kCheckFinite),
                           item("dv_blk", dv_blk, kv, RA_FP32, kCheckFinite)};
  return run_checks(out, 3, hs, "ra_step_bwd", "after the step", RA_ERR_NONFINITE);
}

ra_status ra_count_nonfinite(const void* x, int64_t n, int32_t dtype, int64_t* count, void* stream) {
  if (!count) return fail(RA_ERR_INVALID_ARGUMENT, "count is NULL");
  if (n < 0) return fail(RA_ERR_INVALID_ARGUMENT, "n must be non-negative");
  if (!dtype_ok(dtype)) return fail(RA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  *count = 0;
  if (n == 0) return RA_OK;
  if (!x) return fail(RA_ERR_INVALID_ARGUMENT, "x is NULL");
  const CheckItem it[] = {item("x", x, n, dtype, kCheckFinite)};
  return run_checks(it, 1, (hipStream_t)stream, "ra_count_nonfinite", "", RA_ERR_NONFINITE, count);
}

ra_status ra_count_nonfinite_noalloc(const void* x, int64_t n, int32_t dtype, int64_t* count, void* stream) {
  if (!count) return fail(RA_ERR_INVALID_ARGUMENT, "count is NULL");
  if (n < 0) return fail(RA_ERR_INVALID_ARGUMENT, "n must be non-negative");
  if (!dtype_ok(dtype)) return fail(RA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  *count = 0;
  if (n == 0) return RA_OK;
  if (!x) return fail(RA_ERR_INVALID_ARGUMENT, "x is NULL");
  unsigned long long* dev = nullptr;
  const hipError_t e = scratch_counters(&dev);
  if (e != hipSuccess) return launch_result(e, "scratch counters");
  const CheckItem it[] = {item("x", x, n, dtype, kCheckFinite)};
  return run_checks_with(dev, it, 1, (hipStream_t)stream, "ra_count_nonfinite_noalloc", "", RA_ERR_NONFINITE,
                         count);
}

}  // extern "C"
