// bf16 ring step on gfx950 matrix cores: fold one K/V chunk into the running
// (o_acc, m, l) state of the local queries.
//
// What is computed follows the pages: scores scale * q.k with the ALiBi term
// -slope * |pos_q - pos_k| (intelliparadigm.com long-context survey, §2.1.2),
// the causal mask pos_k <= pos_q on global positions (digipub.cc
// "Zig Zag Ring Attention"), and the tiled online softmax of the same survey's
// §3.1.2 (FlashAttention的核心算法), with the old state rescaled by
// exp(m_old - m_new) and every term taken against the same reference max.
//
// How it maps onto the MI355X:
//  * One 256-thread work-group (4 waves) owns 128 query rows of one head;
//    each wave owns 32 rows. K/V stream through a double-buffered LDS tile of
//    64 keys, moved global -> LDS by the DMA path (global_load_lds_dwordx4, no
//    register staging) while the previous tile is computed; one barrier per
//    tile. Rows past the end of the chunk are clamped to the last key and
//    masked.
//  * The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every
//    lane holds the scores of ONE query (its column) against 16 keys of a
//    32-key block. Row max needs one cross-half exchange (v_permlane32_swap);
//    row sums stay per lane until the end. The rows of the K operand are
//    permuted (bits 2 and 3 of the row index swapped) so that each lane's 16
//    score registers are two runs of 8 consecutive keys -- exactly the B
//    operand layout of the next product.
//  * O^T += V^T P^T, again with the 32x32x16 MFMA: P^T comes straight from
//    the score registers (rounded to bf16); the V^T fragments are read from
//    the row-major V tile with ds_read_b64_tr_b16, whose 16-lane transpose
//    turns "lane j' addresses V[k0 + j'/4][d0 + 4*(j'%4)]" into "lane j holds
//    V[k0 .. k0+3][d0 + j]". The output accumulator keeps one query per lane.
//  * The output is rescaled lazily: exponents are taken against a reference
//    max that is raised (and O, l rescaled) only when a score exceeds it by
//    more than 2^8; P then stays below 2^8, well inside bf16 / fp32 range. The
//    true running max is tracked alongside, and the state is renormalised to
//    it once before it is written, so memory holds exactly m = max s,
//    l = sum exp(s - m), o_acc = sum exp(s - m) v.
//  * Scores are kept in base-2 units (scale * log2 e folded into one FMA) and
//    exponentiated with v_exp_f32; state in memory is in natural units.
//  * Tile classes, all chosen with wave-uniform scalar branches: key tiles
//    past the last query of the work-group are never visited (positions
//    increase); a wave skips tiles entirely in its causal future; tiles that
//    every row of the wave sees in full take the fast path (raw row max, one
//    FMA + one exp per score); only tiles across the diagonal or past the end
//    of the chunk are masked per element. Under the causal mask the ALiBi term
//    of a fully visible tile is linear in the key position, so it becomes one
//    per-key term staged in LDS plus one per-row constant.
//  * Work-groups are ordered heaviest-first and, when the counts allow, each
//    XCD is given whole heads so that its L2 serves one head's K/V stream.
//  * LDS rows are XOR-swizzled in 16-byte units so that the fragment reads of
//    a wave hit distinct banks.
#include <type_traits>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int BM = 128;  // query rows per work-group
constexpr int BN = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, base-2 units

enum TileMode { kFast = 0, kAlibiLinear = 1, kExact = 2 };

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short ra_s16x4;

// K-operand row permutation: swap bits 2 and 3 of a row index in [0, 32).
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// 16-byte chunk swizzles of the K and V rows in LDS.
__device__ __forceinline__ int k_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 1; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, float a0, float a1,
                                            float a2, float a3) {
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  u32x4 v = {__float_as_uint(a0), __float_as_uint(a1), __float_as_uint(a2), __float_as_uint(a3)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (lds_void*)lds_base, 16, 0, 0);
}
// Transposing LDS read, 4 bf16 per lane (see the header comment).
__device__ __forceinline__ uint2 lds_tr4(const void* p) {
  const ra_s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) ra_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(uint2, r);
}

template <int D, bool ALIBI>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(StepArgs a, int n_qtiles,
                                                                int xcd_remap) {
  constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  constexpr int KK = D / 16;            // k-steps of the QK product
  constexpr int DT = D / 32;            // 32-row d tiles of O^T
  constexpr int SLOTS = BN * CPR;       // 16-byte slots in a K (or V) tile
  constexpr int DMA_PER_WAVE = SLOTS / (4 * 64);

  __shared__ uint4 Ks[2][SLOTS];
  __shared__ uint4 Vs[2][SLOTS];
  __shared__ __align__(16) int kp[2][BN];
  __shared__ __align__(16) float kb[ALIBI ? 2 : 1][BN];

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
  const int wave = uniform(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int q0 = qt * BM, q0w = q0 + wave * 32;
  const int row = q0w + l32;
  const bool row_ok = row < Lq;
  const bool wave_active = q0w < Lq;

  const int64_t qhead = (int64_t)b * a.heads_q + h;
  const int64_t khead = (int64_t)b * a.heads_kv + hk;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + khead * Lkv * D;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + khead * Lkv * D;
  const auto rq = make_rsrc(static_cast<const uint16_t*>(a.q) + qhead * Lq * D, (int64_t)Lq * D * 2);
  const auto ro = make_rsrc(a.o_acc + qhead * Lq * D, (int64_t)Lq * D * 4);
  float* mh = a.m + qhead * Lq;
  float* lh = a.l + qhead * Lq;
  const int* kpos = a.k_pos;
  const bool causal = a.causal != 0;

  const int qmax_wg = a.q_pos[min(q0 + BM - 1, Lq - 1)];
  auto tile_live = [&](int kv0) { return kv0 < Lkv && (!causal || kpos[kv0] <= qmax_wg); };
  if (!tile_live(0)) return;  // nothing visible: the state is unchanged

  const int qmin_w = wave_active ? a.q_pos[q0w] : INT32_MAX;
  const int qmax_w = wave_active ? a.q_pos[min(q0w + 31, Lq - 1)] : INT32_MIN;
  const int my_pos = row_ok ? a.q_pos[row] : INT32_MAX;
  const float c = a.scale * RA_LOG2E;
  const bool fast_ok = c > 0.0f;
  const float sl2 = ALIBI ? a.slopes[h] * RA_LOG2E : 0.0f;

  // ---- tile movement: K and V global -> LDS (swizzled), positions via registers ----
  // Slot p of a tile holds row p / CPR, physical chunk p % CPR, i.e. logical
  // chunk (p % CPR) ^ swizzle(row). Each wave moves DMA_PER_WAVE x 64 slots.
  auto dma_tile = [&](int buf, int kv0) {
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int base = (wave * DMA_PER_WAVE + i) * 64;
      const int p = base + lane;
      const int r = p / CPR, ph = p % CPR;
      const int grow = min(kv0 + r, Lkv - 1);
      dma16(kh + (int64_t)grow * D + 8 * (ph ^ k_swz(r)), &Ks[buf][base]);
      dma16(vh + (int64_t)grow * D + 8 * (ph ^ v_swz(r)), &Vs[buf][base]);
    }
  };
  auto load_kp = [&](int kv0) { return tid < BN ? kpos[min(kv0 + tid, Lkv - 1)] : 0; };
  auto store_kp = [&](int buf, int kv0, int kpv) {
    if (tid < BN) {
      kp[buf][tid] = kpv;
      if constexpr (ALIBI) kb[buf][tid] = sl2 * (float)(kpv - kpos[kv0]);
    }
  };

  // Q fragments (B operand of S^T = K Q^T): lane holds query `row`, d slice
  // 16*kk + 8*hf .. +7.
  uint4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = buf_load16(rq, (uint32_t)(row * D + 16 * kk + 8 * hf) * 2);

  // Running state. O^T element (dt, e) of this lane is d = 32*dt + 8*(e/4) +
  // 4*hf + e%4 of query `row`. m_ref: reference max for the exponents; m_max:
  // true running max (both base 2). l per half-wave.
  ra_f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const uint4 v = buf_load16(ro, (uint32_t)(row * D + 32 * dt + 8 * a4 + 4 * hf) * 4);
      O[dt][4 * a4 + 0] = __uint_as_float(v.x);
      O[dt][4 * a4 + 1] = __uint_as_float(v.y);
      O[dt][4 * a4 + 2] = __uint_as_float(v.z);
      O[dt][4 * a4 + 3] = __uint_as_float(v.w);
    }
  }
  float m_ref = row_ok ? mh[row] * RA_LOG2E : -INFINITY;
  float m_max = m_ref;
  float l_run = (row_ok && hf == 0) ? lh[row] : 0.0f;
  bool touched = false;

  // S^T block sb (32 keys) of the tile in LDS buffer `buf`.
  auto qk = [&](int buf, int sb) {
    ra_f32x16 S = ra_f32x16{};
    const int krow = 32 * sb + perm_row(l32);
    const int sw = k_swz(krow);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) S = ra_mfma32(Ks[buf][krow * CPR + ((2 * kk + hf) ^ sw)], qf[kk], S);
    return S;
  };

  // V^T fragment for d tile dt and keys kb0 + 8*hf + 0..7 (two transposing reads).
  const int g16 = lane >> 4, j16 = lane & 15;
  auto v_frag = [&](int buf, int kb0, int dt) {
    const int d0 = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3);
    uint2 r2[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r = kb0 + 8 * hf + 4 * half + (j16 >> 2);
      const int ch = (d0 >> 3) ^ v_swz(r);
      r2[half] = lds_tr4(reinterpret_cast<const char*>(&Vs[buf][r * CPR + ch]) + 2 * (d0 & 7));
    }
    return make_uint4(r2[0].x, r2[0].y, r2[1].x, r2[1].y);
  };

  // Scores of one 32-key block, in place (lane element e is key 32*sb +
  // 16*(e/8) + 8*hf + e%8 of the tile); returns the lane's partial max.
  // kFast leaves raw dot products (the scale is folded into the exponent
  // later); the other modes leave base-2 scores without the per-row ALiBi
  // constant; masked scores are -inf.
  auto scores = [&](auto mode_tag, ra_f32x16& S, int buf, int sb, int kv0) {
    constexpr int MODE = decltype(mode_tag)::value;
    if constexpr (MODE == kAlibiLinear) {
      const float4* kbv = reinterpret_cast<const float4*>(&kb[buf][32 * sb + 8 * hf]);
#pragma unroll
      for (int e8 = 0; e8 < 2; ++e8) {
        const float4 x0 = kbv[4 * e8], x1 = kbv[4 * e8 + 1];
        const float kv8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) S[8 * e8 + i] = fmaf(S[8 * e8 + i], c, kv8[i]);
      }
    } else if constexpr (MODE == kExact) {
      const int4* kpv = reinterpret_cast<const int4*>(&kp[buf][32 * sb + 8 * hf]);
#pragma unroll
      for (int e8 = 0; e8 < 2; ++e8) {
        const int4 p0 = kpv[4 * e8], p1 = kpv[4 * e8 + 1];
        const int kv8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 32 * sb + 16 * e8 + 8 * hf + i;
          float x = S[8 * e8 + i] * c;
          if (ALIBI) x = fmaf(-sl2, (float)abs(my_pos - kv8[i]), x);
          const bool vis = (kv0 + j < Lkv) && (!causal || kv8[i] <= my_pos);
          S[8 * e8 + i] = vis ? x : -INFINITY;
        }
      }
    }
    float t = S[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) t = fmaxf(t, S[e]);
    return t;
  };

  // exp2, row sum and bf16 packing of one block, then O^T += V^T P^T.
  auto pv = [&](auto mode_tag, const ra_f32x16& S, float off, int buf, int sb) {
    constexpr int MODE = decltype(mode_tag)::value;
    uint32_t P[8];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float x0, x1;
      if constexpr (MODE == kFast) {
        x0 = fmaf(S[e], c, off);
        x1 = fmaf(S[e + 1], c, off);
      } else {
        x0 = S[e] + off;
        x1 = S[e + 1] + off;
      }
      const float p0 = __builtin_amdgcn_exp2f(x0);
      const float p1 = __builtin_amdgcn_exp2f(x1);
      psum += p0 + p1;
      P[e >> 1] = ra_pack_bf16(p0, p1);
    }
    l_run += psum;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pb = make_uint4(P[4 * ks + 0], P[4 * ks + 1], P[4 * ks + 2], P[4 * ks + 3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] = ra_mfma32(v_frag(buf, 32 * sb + 16 * ks, dt), pb, O[dt]);
    }
  };

  // One 64-key tile: both score blocks, one row max, one lazy-rescale
  // decision, then the two P.V products.
  auto tile = [&](auto mode_tag, int buf, int kv0) {
    constexpr int MODE = decltype(mode_tag)::value;
    ra_f32x16 S0 = qk(buf, 0);
    ra_f32x16 S1 = qk(buf, 1);
    float tmax = fmaxf(scores(mode_tag, S0, buf, 0, kv0), scores(mode_tag, S1, buf, 1, kv0));
    tmax = fmaxf(tmax, ra_swap_halves(tmax));
    float rowc = 0.0f;  // per-row additive term of kAlibiLinear
    if constexpr (MODE == kFast) {
      tmax *= c;
    } else if constexpr (MODE == kAlibiLinear) {
      // bias = -slope*(pos_q - pos_k) = slope*(pos_k - base) - slope*(pos_q - base)
      rowc = -sl2 * (float)(my_pos - uniform(kpos[kv0]));
      tmax += rowc;
    }
    m_max = fmaxf(m_max, tmax);
    // Lazy rescale: only when a score exceeds the reference by more than 2^tau.
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kTau)) {
      const float nref = fmaxf(m_ref, tmax);
      const float alpha = nref == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref - nref);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
      l_run *= alpha;
      m_ref = nref;
    }
    const float off = rowc - (m_ref == -INFINITY ? 0.0f : m_ref);
    pv(mode_tag, S0, off, buf, 0);
    pv(mode_tag, S1, off, buf, 1);
  };

  // ---- prologue: tile 0 into LDS buffer 0 ----
  dma_tile(0, 0);
  store_kp(0, 0, load_kp(0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kv0 = 0, t = 0;; kv0 += BN, ++t) {
    const int buf = t & 1;
    const bool have_next = tile_live(kv0 + BN);
    int kp_next = 0;
    if (have_next) {  // that buffer was last read before the previous barrier
      dma_tile(buf ^ 1, kv0 + BN);
      kp_next = load_kp(kv0 + BN);
    }

    const int kfirst = uniform(kp[buf][0]);
    const int klast = uniform(kp[buf][BN - 1]);
    if (wave_active && !(causal && kfirst > qmax_w)) {
      touched = true;
      const bool masked = (kv0 + BN > Lkv) || (causal && klast > qmin_w) || !fast_ok;
      if (masked || (ALIBI && !causal))
        tile(std::integral_constant<int, kExact>{}, buf, kv0);
      else if (ALIBI)
        tile(std::integral_constant<int, kAlibiLinear>{}, buf, kv0);
      else
        tile(std::integral_constant<int, kFast>{}, buf, kv0);
    }
    if (!have_next) break;
    store_kp(buf ^ 1, kv0 + BN, kp_next);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA into the other buffer has landed
    __syncthreads();
  }

  if (!touched) return;
  // Renormalise to the true running max and write the state back.
  float l_tot = l_run + ra_swap_halves(l_run);
  const float fac = m_max == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_max);
  l_tot *= fac;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      buf_store16(ro, (uint32_t)(row * D + 32 * dt + 8 * a4 + 4 * hf) * 4, O[dt][4 * a4 + 0] * fac,
                  O[dt][4 * a4 + 1] * fac, O[dt][4 * a4 + 2] * fac, O[dt][4 * a4 + 3] * fac);
    }
  }
  if (row_ok && hf == 0) {
    mh[row] = m_max * RA_LN2;
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
