/*
 * ra.h -- C ABI of libra.so: one ring rank's share of causal blockwise
 * attention on an AMD Instinct MI355X (gfx950).
 *
 * Ring Attention / context parallelism splits a sequence of S tokens over N
 * devices. Each device keeps its query chunk, attends with the K/V chunk it
 * holds, then receives the chunk of device i-1 and passes its own to i+1,
 * until every query has met every key (discosf.com article, §3.1 环形通信拓扑;
 * digipub.cc "大模型如何訓練百萬 Token 上下文", section "Zig Zag Ring
 * Attention"). This library is the work one device does per received chunk:
 * fold the chunk into running max / sum / output accumulators by an online
 * softmax (intelliparadigm.com long-context survey, §3.1.2
 * FlashAttention的核心算法), with the causal mask and an optional ALiBi bias
 * (same survey, §2.1.2) both driven by GLOBAL token positions, so the
 * contiguous split (discosf.com, §2.1 序列切分策略对比) and the zig-zag
 * assignment (token i -> rank i mod N, digipub.cc section above) give the same
 * attention.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *    The compute entry points allocate no device memory and keep no mutable
 *    global state besides the thread-local error text; calls from several
 *    host threads are safe. Only the optional checks below (and
 *    ra_count_nonfinite) hold a small device counter array for the length of
 *    the call.
 *  - Tensors are dense and row-major in the order written: [B, H, L, D] has D
 *    fastest. Positions are int32 and shared by all batches and heads.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    runs asynchronously: RA_OK means "validated and enqueued".
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched and ra_last_error() describes the problem.
 *  - A dimension of zero (empty batch, heads or lengths) is valid and
 *    enqueues nothing.
 *  - Optional checks, switched on per process by environment variables read
 *    at every call (unset or "0" = off). Both make the call wait for its
 *    stream.
 *      RA_CHECK_FINITE=1: ra_step_fwd, ra_finalize, ra_bwd_delta, ra_step_bwd
 *        and ra_rope check that their tensor inputs are finite before
 *        enqueuing any work (a corrupted chunk then leaves the state
 *        untouched) and that their outputs are finite afterwards (m and lse
 *        may be -Inf, l must not be negative), returning RA_ERR_NONFINITE
 *        with the tensor named in ra_last_error(). A ring hands every chunk
 *        from device to device, and a corrupted transfer shows up as NaN or
 *        Inf in what a rank receives (discosf.com article, §5.2 典型问题排查).
 *      RA_DEBUG=1: ra_step_fwd and ra_step_bwd check the precondition that
 *        q_pos and k_pos are non-negative and strictly increasing, returning
 *        RA_ERR_INVALID_ARGUMENT before any launch if they are not.
 */
#ifndef RA_H
#define RA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, negative size, bad enum, inconsistent shape */
  RA_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement (e.g. head_dim) */
  RA_ERR_HIP = 3,              /* the HIP runtime reported an error on launch */
  RA_ERR_NONFINITE = 4         /* a checked tensor holds NaN or Inf (RA_CHECK_FINITE=1) */
} ra_status;

typedef enum ra_dtype { RA_BF16 = 0, RA_FP32 = 1 } ra_dtype;

typedef enum ra_layout {
  RA_CONTIGUOUS = 0, /* rank r holds tokens [r*C, (r+1)*C) */
  RA_ZIGZAG = 1      /* rank r holds tokens r, r+N, r+2N, ... (token i -> rank i mod N) */
} ra_layout;

/* Shapes of one attention step. len_q is the local query chunk length, len_kv
 * the length of the K/V chunk being folded in. heads_q must be a multiple of
 * heads_kv; query head h reads key/value head h / (heads_q / heads_kv).
 * head_dim: 64 or 128 for RA_BF16; 1..128 for RA_FP32. */
typedef struct ra_dims {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  int32_t len_q;
  int32_t len_kv;
  int32_t dtype; /* ra_dtype of q, k, v, o and d_o */
} ra_dims;

/* Global positions of the tokens rank `rank` holds, in local row order
 * (increasing), for a sequence of seq_len tokens over n_ranks ranks:
 * contiguous r*C + t, zig-zag t*N + r, with C = seq_len / n_ranks
 * (discosf.com §2.1; digipub.cc "Zig Zag Ring Attention").
 * rank = -1 writes all ranks: pos_out is int32 [n_ranks, C]; otherwise [C].
 * Errors: seq_len not a positive multiple of n_ranks, seq_len/n_ranks or
 * seq_len above INT32_MAX, bad layout or rank, pos_out NULL. */
ra_status ra_positions(int64_t seq_len, int32_t n_ranks, int32_t rank, int32_t layout,
                       int32_t* pos_out, void* stream);

/* Layout permutation between global sequence order and rank-major chunks.
 * `outer` independent slabs (B*H for a [B,H,S,D] tensor) of seq_len rows of
 * row_elems elements of `dtype` each.
 *   inverse = 0: src is global [outer, S, row]; dst is [n_ranks, outer, C, row]
 *                when rank = -1, or [outer, C, row] holding only that rank;
 *                dst[r][o][t] = src[o][pos_r(t)].
 *   inverse = 1: the reverse gather; src is rank-major ([n_ranks, outer, C,
 *                row], or [outer, C, row] for one rank) and dst is global
 *                [outer, S, row]; with rank >= 0 only that rank's rows of dst
 *                are written.
 * pos (may be NULL) also receives the positions as ra_positions writes them.
 * src and dst must not overlap. Pure data movement: bit-exact. */
ra_status ra_layout_permute(const void* src, void* dst, int32_t* pos, int64_t outer,
                            int64_t seq_len, int32_t row_elems, int32_t dtype, int32_t n_ranks,
                            int32_t layout, int32_t rank, int32_t inverse, void* stream);

/* Rotary position embedding (intelliparadigm.com long-context survey, §2.1.3
 * RoPE的旋转位置编码), applied to `outer` independent slabs of len rows of
 * head_dim elements: x and y are [outer, len, head_dim] in `dtype`. In each
 * row, element j of the first half pairs with element j of the second half
 * (d = head_dim, a = pos[t] * base^(-2j/d)):
 *   y[j] = x[j] cos a - x[j + d/2] sin a,   y[j + d/2] = x[j] sin a + x[j + d/2] cos a.
 * pos: int32 [len], the GLOBAL positions of the rows (non-negative), e.g. the
 * output of ra_positions for a rank's chunk, so either layout gets the rotation
 * its tokens have in the whole sequence; it is shared by all slabs.
 * The angle is reduced exactly (in double precision) and the rotation done in
 * fp32; bf16 results round to nearest even. y may be x (in place) but may not
 * overlap it otherwise. Errors: head_dim odd or outside [2, 256], base not
 * positive and finite, NULL pointers when there is work, unknown dtype. */
ra_status ra_rope(const void* x, void* y, const int32_t* pos, int64_t outer, int64_t len,
                  int32_t head_dim, int32_t dtype, float base, void* stream);

/* Start state of the running accumulators: o_acc = 0 [B,Hq,Lq,D], m = -inf and
 * l = 0 [B,Hq,Lq] (the initial max and sum of the online softmax,
 * intelliparadigm.com §3.1.2). All fp32. Only batch, heads_q, head_dim and
 * len_q of d are used. */
ra_status ra_state_init(const ra_dims* d, float* o_acc, float* m, float* l, void* stream);

/* One ring step: fold the K/V chunk (k_blk, v_blk: [B, Hkv, Lkv, D]) into the
 * running state of the local queries q [B, Hq, Lq, D].
 *
 * Scores are s = scale * <q_i, k_j> - slope_h * |q_pos[i] - k_pos[j]| (the
 * ALiBi term only when alibi_slopes != NULL, alibi_slopes being fp32 [Hq]);
 * with causal != 0 a key is visible only if k_pos[j] <= q_pos[i].
 * The state, all fp32 and updated in place, is defined over the keys J folded
 * in so far: m is the reference of the exponentials, l = sum_J exp(s - m) and
 * o_acc = sum_J exp(s - m) v_j (natural exponent), so that m + ln l is the
 * log-sum-exp of the row and o_acc / l its output whatever m is. The fp32
 * path keeps m = max_J s; the bf16 path moves m only when the scores outgrow
 * it, so that max_J s - 14 ln 2 <= m <= max_J s (and l >= 1). Rows with no
 * visible key keep m = -inf, l = 0, o_acc = 0. Chunks may be folded in any
 * order; the result differs only by rounding.
 * q_pos [Lq] and k_pos [Lkv] must be strictly increasing (both layouts give
 * that); tiles that are masked out entirely are skipped using this.
 * Positions must be non-negative. For bf16, q, k_blk, v_blk and o_acc must be
 * 16-byte aligned (RA_ERR_INVALID_ARGUMENT otherwise).
 * Size limits (RA_ERR_UNSUPPORTED beyond them, checked before any launch):
 * bf16 addresses one head's o_acc slab through a 32-bit buffer resource, so
 * len_q * head_dim * 4 must stay below 2^31 (len_q <= 4,194,303 at
 * head_dim 128); the number of work-groups (one per 128 rows of a head, bf16,
 * or 32 rows, fp32, at most) must fit in int32.
 * Computation: bf16 inputs use bf16 MFMA with fp32 accumulation (P is rounded
 * to bf16 before the P.V product); fp32 inputs are computed in fp32. */
ra_status ra_step_fwd(const ra_dims* d, const void* q, const void* k_blk, const void* v_blk,
                      const int32_t* q_pos, const int32_t* k_pos, int32_t causal, float scale,
                      const float* alibi_slopes, float* o_acc, float* m, float* l, void* stream);

/* Normalise after the last step: o = o_acc / l in d->dtype (bf16 round to
 * nearest even) and lse = m + ln(l) in fp32 (intelliparadigm.com §3.1.2, the
 * final division by l). Rows with l = 0 give o = 0 and lse = -inf.
 * o: [B,Hq,Lq,D]; lse: [B,Hq,Lq]; either may be NULL to skip it. */
ra_status ra_finalize(const ra_dims* d, const float* o_acc, const float* m, const float* l,
                      void* o, float* lse, void* stream);

/* Backward pre-pass, once per ring pass: delta[i] = sum_d d_o[i,d] * o[i,d]
 * (fp32 [B,Hq,Lq]), the row term of the softmax gradient. o and d_o are
 * [B,Hq,Lq,D] in d->dtype. */
ra_status ra_bwd_delta(const ra_dims* d, const void* o, const void* d_o, float* delta,
                       void* stream);

/* One backward ring step for the K/V chunk (k_blk, v_blk). The pages only say
 * that the backward recomputes attention from saved statistics instead of
 * storing it (intelliparadigm.com §3.1.2); the gradients are the textbook
 * ones, with P recomputed from the final lse of ra_finalize:
 *   P = exp(s - lse), dS = P * (d_o . v^T - delta),
 *   dq_acc += scale * dS k,  dk_blk += scale * dS^T q,  dv_blk += P^T d_o.
 * Same masking, positions and ALiBi term as ra_step_fwd. dq_acc
 * [B,Hq,Lq,D], dk_blk and dv_blk [B,Hkv,Lkv,D] are fp32 and ACCUMULATE
 * (caller zeroes them once); query heads sharing a K/V head add into it.
 * Supported for RA_BF16 with head_dim 128 (bf16 matrix-core products with
 * fp32 accumulation; P and dS are rounded to bf16 before their products) and
 * for RA_FP32 with head_dim 1..128 (computed in fp32 throughout: the
 * correctness path). Deterministic (no atomics).
 * Size limits (RA_ERR_UNSUPPORTED beyond them): for bf16 one head's q / d_o
 * slab and k / v slab must stay below 2^31 bytes (len_q, len_kv <= 8,388,607
 * at head_dim 128); the work-group count must fit in int32. */
ra_status ra_step_bwd(const ra_dims* d, const void* q, const void* k_blk, const void* v_blk,
                      const int32_t* q_pos, const int32_t* k_pos, int32_t causal, float scale,
                      const float* alibi_slopes, const void* d_o, const float* lse,
                      const float* delta, float* dq_acc, float* dk_blk, float* dv_blk,
                      void* stream);

/* Number of NaN or Inf elements among the n elements of x (a device tensor
 * of `dtype`), counted on the GPU on `stream`; the call waits for the count
 * and writes it to *count (host memory). Lets a caller check a chunk it has
 * received before folding it in (discosf.com article, §5.2 典型问题排查: a
 * ring transfer may corrupt data). Holds a small device counter array,
 * allocated and freed inside the call. Errors: count NULL, n negative, x NULL
 * with n > 0, unknown dtype. */
ra_status ra_count_nonfinite(const void* x, int64_t n, int32_t dtype, int64_t* count, void* stream);

/* ra_count_nonfinite without any allocation, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid it).
 * Same arguments, result and errors. Its counter lives in a 64-byte static
 * device array of the library (one copy per GPU, held until the process
 * ends, found through hipGetSymbolAddress once per device), not in memory
 * allocated per call; n may take any value, since one 64-bit counter serves
 * any size. Every call on a GPU shares that array, which is cleared at the
 * start of each call: calls that overlap on one GPU (several host threads,
 * or streams running concurrently) race and may return wrong counts. Uses
 * the current device; `stream` must belong to it. */
ra_status ra_count_nonfinite_noalloc(const void* x, int64_t n, int32_t dtype, int64_t* count,
                                     void* stream);

/* Text for the last non-OK status returned on this host thread ("" if none). */
const char* ra_last_error(void);

/* Version of this library's ABI (increments on incompatible change). */
int32_t ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
