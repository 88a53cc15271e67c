// bf16 ring step on gfx950 matrix cores: fold one K/V chunk into the running
// (o_acc, m, l) state of the local queries.
//
// What is computed follows the pages: scores scale * q.k with the ALiBi term
// -slope * |pos_q - pos_k| (intelliparadigm.com long-context survey, §2.1.2),
// the causal mask pos_k <= pos_q on global positions (digipub.cc
// "Zig Zag Ring Attention"), and the tiled online softmax of the same survey's
// §3.1.2 (FlashAttention的核心算法) with the old state rescaled by
// exp(m_old - m_new) and the tile's terms taken against that same m_new.
//
// How it maps onto the MI355X:
//  * One 256-thread work-group (4 waves) owns 128 query rows of one head;
//    each wave owns 32 rows. K/V are streamed through LDS 64 keys at a time.
//  * The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every
//    lane holds the scores of ONE query (its column) against 16 keys per
//    32-key block. Row max needs one cross-half exchange (v_permlane32_swap);
//    row sums stay per lane until the end. The rows of the K operand are
//    permuted (bits 2 and 3 of the row index swapped) so that each lane's 16
//    score registers are two runs of 8 consecutive keys -- exactly the B
//    operand layout of the next product.
//  * O^T += V^T P^T, again with the 32x32x16 MFMA: P^T comes straight from
//    the score registers (rounded to bf16), V^T is read from an LDS copy of V
//    stored transposed, and the output accumulator keeps one query per lane,
//    so the rescale by exp(m_old - m_new) is a per-lane scalar.
//  * Q stays in registers for the whole chunk. The next K/V tile is fetched
//    into registers while the current one is computed.
//  * Scores are kept in base-2 units (scale * log2 e folded into one FMA) and
//    exponentiated with v_exp_f32; state in memory is in natural units.
//  * Key tiles past the last query of the work-group are never visited
//    (positions increase), tiles entirely below every query of a wave need
//    no mask, and only the few tiles across the diagonal are masked per
//    element. Work-groups are ordered heaviest-first and, when the counts
//    allow, each XCD is given whole heads so that its L2 serves one head's K/V.
//  * LDS rows are XOR-swizzled in 16-byte units so that the fragment reads of
//    a wave hit distinct banks.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int BM = 128;  // query rows per work-group
constexpr int BN = 64;   // keys per tile
constexpr int kThreads = 256;

// K-operand row permutation: swap bits 2 and 3 of a row index in [0, 32).
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// Swizzle of the 16-byte chunk index within a K row of the LDS tile.
__device__ __forceinline__ int k_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

template <int D, bool ALIBI>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(StepArgs a, int n_qtiles,
                                                                int xcd_remap) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int KK = D / 16;                 // k-steps of the QK product
  constexpr int DT = D / 32;                 // 32-row d tiles of O^T
  constexpr int RPP = kThreads / CPR;        // K rows loaded per pass
  constexpr int KPASS = BN / RPP;            // passes for a K tile
  constexpr int VBLK = (BN / 4) * CPR;       // 4x8 transpose blocks in a V tile
  constexpr int VCH = BN / 8;                // 16-byte chunks per V^T row

  __shared__ uint4 Ks[BN * CPR];
  __shared__ uint4 Vt[D * VCH];
  __shared__ int kp[BN];

  const int Lq = a.len_q, Lkv = a.len_kv;
  const int BH = a.batch * a.heads_q;
  int task = blockIdx.x;
  if (xcd_remap) {
    const int per = (n_qtiles * BH) >> 3;
    task = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  const int bh = task / n_qtiles;
  const int qt = n_qtiles - 1 - (task - bh * n_qtiles);
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int q0 = qt * BM, q0w = q0 + wave * 32;
  const int row = q0w + l32;
  const bool row_ok = row < Lq;
  const bool wave_active = q0w < Lq;

  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.heads_q + h) * Lq * D;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + ((int64_t)b * a.heads_kv + hk) * Lkv * D;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + ((int64_t)b * a.heads_kv + hk) * Lkv * D;
  float* oh = a.o_acc + ((int64_t)b * a.heads_q + h) * Lq * D;
  float* mh = a.m + ((int64_t)b * a.heads_q + h) * Lq;
  float* lh = a.l + ((int64_t)b * a.heads_q + h) * Lq;
  const int* kpos = a.k_pos;
  const bool causal = a.causal != 0;

  const int qmax_wg = a.q_pos[min(q0 + BM - 1, Lq - 1)];
  auto tile_live = [&](int kv0) { return kv0 < Lkv && (!causal || kpos[kv0] <= qmax_wg); };
  if (!tile_live(0)) return;  // nothing visible: the state is unchanged

  const int qmin_w = wave_active ? a.q_pos[q0w] : INT32_MAX;
  const int qmax_w = wave_active ? a.q_pos[min(q0w + 31, Lq - 1)] : INT32_MIN;
  const int my_pos = row_ok ? a.q_pos[row] : INT32_MAX;
  const float c = a.scale * RA_LOG2E;
  const bool raw_max = !ALIBI && c > 0.0f;  // max of raw scores, scaled afterwards
  const float sl2 = ALIBI ? a.slopes[h] * RA_LOG2E : 0.0f;

  // Q fragments (B operand of S^T = K Q^T): lane holds query `row`, d slice
  // 16*kk + 8*hf .. +7.
  uint4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = row_ok ? *reinterpret_cast<const uint4*>(qh + (int64_t)row * D + 16 * kk + 8 * hf)
                    : make_uint4(0, 0, 0, 0);

  // Running state. O^T element (dt, e) of this lane is d = 32*dt + 8*(e/4) +
  // 4*hf + e%4 of query `row`. m is kept in base-2 units, l per half-wave.
  ra_f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      float4 v = row_ok ? *reinterpret_cast<const float4*>(oh + (int64_t)row * D + 32 * dt + 8 * a4 + 4 * hf)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
      O[dt][4 * a4 + 0] = v.x;
      O[dt][4 * a4 + 1] = v.y;
      O[dt][4 * a4 + 2] = v.z;
      O[dt][4 * a4 + 3] = v.w;
    }
  }
  float m_run = row_ok ? mh[row] * RA_LOG2E : -INFINITY;
  float l_run = (row_ok && hf == 0) ? lh[row] : 0.0f;
  bool touched = false;

  // Register staging of the next tile.
  uint4 kreg[KPASS];
  uint4 vreg[4];
  int kpreg = INT32_MAX;
  const int kc = tid % CPR, kr = tid / CPR;           // K: chunk, first row
  const int vdc = tid % CPR, vkv4 = tid / CPR;        // V: d chunk, 4-key group

  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int r = kr + i * RPP;
      kreg[i] = kv0 + r < Lkv ? *reinterpret_cast<const uint4*>(kh + (int64_t)(kv0 + r) * D + 8 * kc)
                              : make_uint4(0, 0, 0, 0);
    }
    if (tid < VBLK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * vkv4 + j;
        vreg[j] = kv0 + r < Lkv ? *reinterpret_cast<const uint4*>(vh + (int64_t)(kv0 + r) * D + 8 * vdc)
                                : make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BN) kpreg = kv0 + tid < Lkv ? kpos[kv0 + tid] : INT32_MAX;
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int r = kr + i * RPP;
      Ks[r * CPR + (kc ^ k_swz(r))] = kreg[i];
    }
    if (tid < VBLK) {
      // 4 keys x 8 dims -> for each dim d, 4 consecutive keys (8 bytes).
      const uint32_t w[4][4] = {{vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w},
                                {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w},
                                {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w},
                                {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w}};
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wi = dd >> 1;
        uint2 out;
        if (dd & 1) {
          out.x = (w[0][wi] >> 16) | (w[1][wi] & 0xffff0000u);
          out.y = (w[2][wi] >> 16) | (w[3][wi] & 0xffff0000u);
        } else {
          out.x = (w[0][wi] & 0xffffu) | (w[1][wi] << 16);
          out.y = (w[2][wi] & 0xffffu) | (w[3][wi] << 16);
        }
        const int d = 8 * vdc + dd;
        const int ch = (vkv4 >> 1) ^ (d & 7);
        reinterpret_cast<uint2*>(&Vt[d * VCH + ch])[vkv4 & 1] = out;
      }
    }
    if (tid < BN) kp[tid] = kpreg;
  };

  int kv0 = 0;
  load_tile(0);
  while (true) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    const int nxt = kv0 + BN;
    const bool has_next = tile_live(nxt);
    if (has_next) load_tile(nxt);

    const bool wave_skip = !wave_active || (causal && kp[0] > qmax_w);
    if (!wave_skip) {
      touched = true;
      const bool need_mask = (kv0 + BN > Lkv) || (causal && kp[BN - 1] > qmin_w);

      // ---- S^T = K Q^T for two 32-key blocks ----
      ra_f32x16 S[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        S[sb] = ra_f32x16{};
        const int krow = 32 * sb + perm_row(l32);
        const int sw = k_swz(krow);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          S[sb] = ra_mfma32(Ks[krow * CPR + ((2 * kk + hf) ^ sw)], qf[kk], S[sb]);
      }
      // Lane element (sb, e) is key 32*sb + 16*(e/8) + 8*hf + e%8 of the tile.

      // ---- scores, mask, row max ----
      bool scaled = !raw_max;
      if (ALIBI || need_mask || !raw_max) {
        scaled = true;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = 32 * sb + 16 * (e >> 3) + 8 * hf + (e & 7);
            float x = S[sb][e] * c;
            if (ALIBI) x = fmaf(-sl2, (float)abs(my_pos - kp[j]), x);
            if (need_mask) {
              const bool vis = (kv0 + j < Lkv) && (!causal || kp[j] <= my_pos);
              x = vis ? x : -INFINITY;
            }
            S[sb][e] = x;
          }
        }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, S[sb][e]);
      mt = fmaxf(mt, ra_swap_halves(mt));
      if (!scaled) mt *= c;

      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      // ---- P = exp2(s - m), row sums, bf16 packing ----
      uint32_t P[2][8];
      float psum = 0.0f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float x0 = scaled ? S[sb][e] - m_use : fmaf(S[sb][e], c, -m_use);
          const float x1 = scaled ? S[sb][e + 1] - m_use : fmaf(S[sb][e + 1], c, -m_use);
          const float p0 = __builtin_amdgcn_exp2f(x0);
          const float p1 = __builtin_amdgcn_exp2f(x1);
          psum += p0 + p1;
          P[sb][e >> 1] = ra_pack_bf16(p0, p1);
        }
      }
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 pb = make_uint4(P[sb][4 * ks + 0], P[sb][4 * ks + 1], P[sb][4 * ks + 2],
                                      P[sb][4 * ks + 3]);
          const int c8 = 4 * sb + 2 * ks + hf;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int d = 32 * dt + l32;
            O[dt] = ra_mfma32(Vt[d * VCH + (c8 ^ (d & 7))], pb, O[dt]);
          }
        }
      }
    }
    if (!has_next) break;
    kv0 = nxt;
  }

  const float l_tot = l_run + ra_swap_halves(l_run);
  if (!touched || !row_ok) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      *reinterpret_cast<float4*>(oh + (int64_t)row * D + 32 * dt + 8 * a4 + 4 * hf) =
          make_float4(O[dt][4 * a4 + 0], O[dt][4 * a4 + 1], O[dt][4 * a4 + 2], O[dt][4 * a4 + 3]);
    }
  }
  if (hf == 0) {
    mh[row] = m_run * RA_LN2;
    lh[row] = l_tot;
  }
}

template <int D, bool ALIBI>
hipError_t launch_d(const StepArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.len_q + BM - 1) / BM;
  const int64_t grid = (int64_t)n_qtiles * a.batch * a.heads_q;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, ALIBI>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     a, n_qtiles, remap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const StepArgs& a, hipStream_t stream) {
  const bool alibi = a.slopes != nullptr;
  if (a.head_dim == 128) return alibi ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  return alibi ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
}

}  // namespace ra
