// fp32 backward ring step: the correctness path of the backward, computed in
// fp32 throughout (no bf16 rounding anywhere), for head_dim 1..128.
//
// The pages only say that the backward recomputes the attention matrix from
// saved statistics instead of storing it (intelliparadigm.com long-context
// survey, §3.1.2, 重计算策略); the gradients are the textbook ones, with the
// forward's scores s = scale * q.k - slope * |pos_q - pos_k| (causal-masked on
// global positions) and the final lse of each query row:
//   P = exp(s - lse),  dS = P * (dO . v - delta),  delta = <dO, O>,
//   dQ_i += scale * sum_j dS_ij k_j,  dK_j += scale * sum_i dS_ij q_i,
//   dV_j += sum_i P_ij dO_i.
// Two deterministic kernels (no atomics; each output element is owned by one
// lane and summed in a fixed order), laid out like the fp32 forward step:
// TPR = ceil(D / 32) lanes share one row, each holding 32 of its elements,
// and the dot products are reduced across those lanes with shuffles.
//  * bwd_dq_fp32_kernel: a block owns ROWS query rows of one head and walks
//    the key chunk in tiles of 32 keys staged in LDS.
//  * bwd_dkdv_fp32_kernel: a block owns ROWS keys of one K/V head and walks
//    every query head of its group and the query rows in tiles of 32.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kThreads = 128;
constexpr int kTile = 32;

__device__ __forceinline__ float lse_shift(float lse) {
  // exp(s - lse) must be 0 for a row that saw no key (lse = -inf).
  return lse == -INFINITY ? INFINITY : lse;
}

template <int DP>
__device__ __forceinline__ float row_dot(const float (&x)[32], const float* y, int dbase) {
  constexpr int TPR = DP / 32;
  float part = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) part = fmaf(x[e], y[dbase + e], part);
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) part += __shfl_xor(part, off, TPR);
  return part;
}

template <int DP>
__global__ __launch_bounds__(kThreads) void bwd_dq_fp32_kernel(BwdArgs a) {
  constexpr int TPR = DP / 32;
  constexpr int ROWS = kThreads / TPR;
  __shared__ float Ks[kTile][DP];
  __shared__ float Vs[kTile][DP];
  __shared__ int kp[kTile];

  const int D = a.head_dim, Lq = a.len_q, Lkv = a.len_kv;
  const int n_rt = (Lq + ROWS - 1) / ROWS;
  const int bh = blockIdx.x / n_rt, rt = blockIdx.x - bh * n_rt;
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
  const int tid = threadIdx.x, sub = tid % TPR, dbase = sub * 32;
  const int row = rt * ROWS + tid / TPR;
  const bool row_ok = row < Lq;

  const int64_t qrow0 = ((int64_t)b * a.heads_q + h) * Lq;
  const float* q = static_cast<const float*>(a.q) + qrow0 * D;
  const float* dout = static_cast<const float*>(a.d_o) + qrow0 * D;
  const float* k = static_cast<const float*>(a.k) + ((int64_t)b * a.heads_kv + hk) * Lkv * D;
  const float* v = static_cast<const float*>(a.v) + ((int64_t)b * a.heads_kv + hk) * Lkv * D;
  const int qmax_blk = a.q_pos[min(rt * ROWS + ROWS - 1, Lq - 1)];
  const int my_pos = row_ok ? a.q_pos[row] : INT32_MAX;
  const float my_lse = row_ok ? lse_shift(a.lse[qrow0 + row]) : INFINITY;
  const float my_del = row_ok ? a.delta[qrow0 + row] : 0.0f;
  const float slope = a.slopes ? a.slopes[h] : 0.0f;

  float qv[32], ov[32], dq[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int d = dbase + e;
    const bool ok = row_ok && d < D;
    qv[e] = ok ? q[(int64_t)row * D + d] : 0.0f;
    ov[e] = ok ? dout[(int64_t)row * D + d] : 0.0f;
    dq[e] = 0.0f;
  }
  bool touched = false;
  for (int kv0 = 0; kv0 < Lkv; kv0 += kTile) {
    if (a.causal && a.k_pos[kv0] > qmax_blk) break;  // positions increase: the rest is masked
    __syncthreads();
    for (int i = tid; i < kTile * DP; i += kThreads) {
      const int j = i / DP, d = i - j * DP;
      const bool ok = kv0 + j < Lkv && d < D;
      Ks[j][d] = ok ? k[(int64_t)(kv0 + j) * D + d] : 0.0f;
      Vs[j][d] = ok ? v[(int64_t)(kv0 + j) * D + d] : 0.0f;
    }
    if (tid < kTile) kp[tid] = kv0 + tid < Lkv ? a.k_pos[kv0 + tid] : INT32_MAX;
    __syncthreads();
    touched = true;
    for (int j = 0; j < kTile; ++j) {
      float s = a.scale * row_dot<DP>(qv, Ks[j], dbase);
      if (a.slopes) s -= slope * (float)abs(my_pos - kp[j]);
      const float dp = row_dot<DP>(ov, Vs[j], dbase);
      const bool vis = kv0 + j < Lkv && (!a.causal || kp[j] <= my_pos);
      const float p = vis ? expf(s - my_lse) : 0.0f;
      const float ds = p * (dp - my_del);
#pragma unroll
      for (int e = 0; e < 32; ++e) dq[e] = fmaf(ds, Ks[j][dbase + e], dq[e]);
    }
  }
  if (!touched || !row_ok) return;
  float* dqr = a.dq + (qrow0 + row) * D;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int d = dbase + e;
    if (d < D) dqr[d] += a.scale * dq[e];
  }
}

template <int DP>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_fp32_kernel(BwdArgs a) {
  constexpr int TPR = DP / 32;
  constexpr int ROWS = kThreads / TPR;
  __shared__ float Qs[kTile][DP];
  __shared__ float Os[kTile][DP];  // dO
  __shared__ float lse_s[kTile], del_s[kTile];
  __shared__ int qp[kTile];

  const int D = a.head_dim, Lq = a.len_q, Lkv = a.len_kv;
  const int g = a.heads_q / a.heads_kv;
  const int n_kt = (Lkv + ROWS - 1) / ROWS;
  const int bh = blockIdx.x / n_kt, kt = blockIdx.x - bh * n_kt;
  const int b = bh / a.heads_kv, hk = bh - b * a.heads_kv;
  const int tid = threadIdx.x, sub = tid % TPR, dbase = sub * 32;
  const int key = kt * ROWS + tid / TPR;
  const bool key_ok = key < Lkv;

  const int64_t krow0 = ((int64_t)b * a.heads_kv + hk) * Lkv;
  const float* k = static_cast<const float*>(a.k) + krow0 * D;
  const float* v = static_cast<const float*>(a.v) + krow0 * D;
  const int kmin_blk = a.k_pos[min(kt * ROWS, Lkv - 1)];
  const int my_kpos = key_ok ? a.k_pos[key] : INT32_MAX;

  float kv_[32], vv[32], dk[32], dv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int d = dbase + e;
    const bool ok = key_ok && d < D;
    kv_[e] = ok ? k[(int64_t)key * D + d] : 0.0f;
    vv[e] = ok ? v[(int64_t)key * D + d] : 0.0f;
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  // First query row that can see a key of this block (positions increase).
  int qstart = 0;
  if (a.causal) {
    int lo = 0, hi = Lq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.q_pos[mid] < kmin_blk) lo = mid + 1; else hi = mid;
    }
    qstart = lo;
  }
  qstart = qstart / kTile * kTile;
  bool touched = false;
  for (int hh = 0; hh < g; ++hh) {
    const int h = hk * g + hh;
    const int64_t qrow0 = ((int64_t)b * a.heads_q + h) * Lq;
    const float* q = static_cast<const float*>(a.q) + qrow0 * D;
    const float* dout = static_cast<const float*>(a.d_o) + qrow0 * D;
    const float slope = a.slopes ? a.slopes[h] : 0.0f;
    for (int q0 = qstart; q0 < Lq; q0 += kTile) {
      __syncthreads();
      for (int i = tid; i < kTile * DP; i += kThreads) {
        const int r = i / DP, d = i - r * DP;
        const bool ok = q0 + r < Lq && d < D;
        Qs[r][d] = ok ? q[(int64_t)(q0 + r) * D + d] : 0.0f;
        Os[r][d] = ok ? dout[(int64_t)(q0 + r) * D + d] : 0.0f;
      }
      if (tid < kTile) {
        const bool ok = q0 + tid < Lq;
        qp[tid] = ok ? a.q_pos[q0 + tid] : INT32_MAX;  // masked by its index; no overflow in |q - k|
        lse_s[tid] = ok ? lse_shift(a.lse[qrow0 + q0 + tid]) : INFINITY;
        del_s[tid] = ok ? a.delta[qrow0 + q0 + tid] : 0.0f;
      }
      __syncthreads();
      touched = true;
      for (int i = 0; i < kTile; ++i) {
        float s = a.scale * row_dot<DP>(kv_, Qs[i], dbase);
        if (a.slopes) s -= slope * (float)abs(qp[i] - my_kpos);
        const float dp = row_dot<DP>(vv, Os[i], dbase);
        const bool vis = q0 + i < Lq && (!a.causal || my_kpos <= qp[i]);
        const float p = vis ? expf(s - lse_s[i]) : 0.0f;
        const float ds = p * (dp - del_s[i]);
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          dv[e] = fmaf(p, Os[i][dbase + e], dv[e]);
          dk[e] = fmaf(ds, Qs[i][dbase + e], dk[e]);
        }
      }
    }
  }
  if (!touched || !key_ok) return;
  float* dkr = a.dk + (krow0 + key) * D;
  float* dvr = a.dv + (krow0 + key) * D;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int d = dbase + e;
    if (d < D) {
      dkr[d] += a.scale * dk[e];
      dvr[d] += dv[e];
    }
  }
}

template <int DP>
hipError_t launch_dp(const BwdArgs& a, hipStream_t stream) {
  constexpr int ROWS = kThreads / (DP / 32);
  const int64_t grid_q = (int64_t)((a.len_q + ROWS - 1) / ROWS) * a.batch * a.heads_q;
  const int64_t grid_k = (int64_t)((a.len_kv + ROWS - 1) / ROWS) * a.batch * a.heads_kv;
  if (grid_q > INT32_MAX || grid_k > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_fp32_kernel<DP>, dim3((unsigned)grid_q), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_fp32_kernel<DP>, dim3((unsigned)grid_k), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_fp32(const BwdArgs& a, hipStream_t stream) {
  const int D = a.head_dim;
  if (D <= 32) return launch_dp<32>(a, stream);
  if (D <= 64) return launch_dp<64>(a, stream);
  return launch_dp<128>(a, stream);
}

}  // namespace ra
