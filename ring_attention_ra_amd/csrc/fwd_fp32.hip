// fp32 ring step: fold one K/V chunk into the running (o_acc, m, l) state of
// the local queries, computed entirely in fp32 FMA arithmetic.
//
// Per key tile the update is the online softmax of intelliparadigm.com
// (long-context survey, §3.1.2 FlashAttention的核心算法) in its correct form:
// the old state is rescaled by exp(m_old - m_new) and the tile's terms are
// taken relative to the same m_new. Scores carry the ALiBi term
// -slope * |pos_q - pos_k| of §2.1.2 of the same survey and the causal mask
// pos_k <= pos_q on global positions (digipub.cc "Zig Zag Ring Attention").
//
// Layout of the work: 128 threads per block; each query row is owned by
// TPR = DP/32 consecutive lanes, each holding a 32-wide slice of q and of the
// output accumulator. Keys are staged through LDS 32 at a time and read as
// broadcasts.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kThreads = 128;
constexpr int kKeys = 32;

template <int DP>
__global__ __launch_bounds__(kThreads) void fwd_fp32_kernel(StepArgs a) {
  constexpr int TPR = DP / 32;              // lanes per query row
  constexpr int ROWS = kThreads / TPR;      // query rows per block
  __shared__ float Ks[kKeys][DP];
  __shared__ float Vs[kKeys][DP];
  __shared__ int kp[kKeys];

  const int D = a.head_dim;
  const int Lq = a.len_q, Lkv = a.len_kv;
  const int n_rt = (Lq + ROWS - 1) / ROWS;
  const int bh = blockIdx.x / n_rt;
  const int rt = blockIdx.x - bh * n_rt;
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
  const int tid = threadIdx.x;
  const int sub = tid % TPR;
  const int row = rt * ROWS + tid / TPR;
  const bool row_ok = row < Lq;
  const int dbase = sub * 32;

  const float* q = static_cast<const float*>(a.q) + ((int64_t)b * a.heads_q + h) * Lq * D;
  const float* k = static_cast<const float*>(a.k) + ((int64_t)b * a.heads_kv + hk) * Lkv * D;
  const float* v = static_cast<const float*>(a.v) + ((int64_t)b * a.heads_kv + hk) * Lkv * D;
  float* oacc = a.o_acc + ((int64_t)b * a.heads_q + h) * Lq * D;
  float* mrow = a.m + ((int64_t)b * a.heads_q + h) * Lq;
  float* lrow = a.l + ((int64_t)b * a.heads_q + h) * Lq;

  const int last = min(rt * ROWS + ROWS - 1, Lq - 1);
  const int qmax_blk = a.q_pos[last];
  const int my_pos = row_ok ? a.q_pos[row] : INT32_MAX;
  const float slope = a.slopes ? a.slopes[h] : 0.0f;

  float qv[32], ov[32];
#pragma unroll
  for (int x = 0; x < 32; ++x) {
    const int d = dbase + x;
    const bool ok = row_ok && d < D;
    qv[x] = ok ? q[(int64_t)row * D + d] : 0.0f;
    ov[x] = ok ? oacc[(int64_t)row * D + d] : 0.0f;
  }
  float m_run = row_ok ? mrow[row] : -INFINITY;
  float l_run = row_ok ? lrow[row] : 0.0f;
  bool touched = false;

  for (int kv0 = 0; kv0 < Lkv; kv0 += kKeys) {
    if (a.causal && a.k_pos[kv0] > qmax_blk) break;  // positions increase: the rest is masked
    __syncthreads();
    for (int i = tid; i < kKeys * DP; i += kThreads) {
      const int j = i / DP, d = i - (i / DP) * DP;
      const bool ok = kv0 + j < Lkv && d < D;
      Ks[j][d] = ok ? k[(int64_t)(kv0 + j) * D + d] : 0.0f;
      Vs[j][d] = ok ? v[(int64_t)(kv0 + j) * D + d] : 0.0f;
    }
    if (tid < kKeys) kp[tid] = kv0 + tid < Lkv ? a.k_pos[kv0 + tid] : INT32_MAX;
    __syncthreads();
    touched = true;

    float s[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float part = 0.0f;
#pragma unroll
      for (int x = 0; x < 32; ++x) part = fmaf(qv[x], Ks[j][dbase + x], part);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) part += __shfl_xor(part, off, TPR);
      float sc = a.scale * part;
      if (a.slopes) sc -= slope * (float)abs(my_pos - kp[j]);
      const bool vis = kv0 + j < Lkv && (!a.causal || kp[j] <= my_pos);
      s[j] = vis ? sc : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = expf(m_run - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int x = 0; x < 32; ++x) ov[x] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m_use);
      psum += p;
#pragma unroll
      for (int x = 0; x < 32; ++x) ov[x] = fmaf(p, Vs[j][dbase + x], ov[x]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
  }

  if (!touched || !row_ok) return;
#pragma unroll
  for (int x = 0; x < 32; ++x) {
    const int d = dbase + x;
    if (d < D) oacc[(int64_t)row * D + d] = ov[x];
  }
  if (sub == 0) {
    mrow[row] = m_run;
    lrow[row] = l_run;
  }
}

}  // namespace

hipError_t launch_fwd_fp32(const StepArgs& a, hipStream_t stream) {
  const int D = a.head_dim;
  const int dp = D <= 32 ? 32 : (D <= 64 ? 64 : 128);
  const int rows = kThreads / (dp / 32);
  const int64_t grid = (int64_t)((a.len_q + rows - 1) / rows) * a.batch * a.heads_q;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  switch (dp) {
    case 32:
      hipLaunchKernelGGL(fwd_fp32_kernel<32>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
    case 64:
      hipLaunchKernelGGL(fwd_fp32_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(fwd_fp32_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ra
