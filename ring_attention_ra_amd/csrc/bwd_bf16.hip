// Backward ring step on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The pages only say that the backward recomputes the attention matrix from
// saved statistics instead of storing it (intelliparadigm.com long-context
// survey, §3.1.2, 重计算策略); the gradients are the textbook ones. With the
// forward's scores s = scale * q.k - slope * |pos_q - pos_k| (causal-masked on
// global positions) and the final lse of each query row:
//   P  = exp(s - lse),   dP = dO . v,   dS = P * (dP - delta),  delta = <dO, O>
//   dV_j += sum_i P_ij dO_i,  dK_j += scale * sum_i dS_ij q_i,
//   dQ_i += scale * sum_j dS_ij k_j.
// Two kernels, both deterministic (no atomics; every output element is owned
// by one lane and accumulated in a fixed order):
//  * bwd_dkdv_kernel: a work-group owns 128 keys (4 waves x 32) of one K/V
//    head and walks every query head of its group and every 64-query tile that
//    sees those keys. K and V fragments stay in registers. S = Q K^T and
//    dP = dO V^T run with the query rows as the MFMA A operand (rows permuted
//    so that each lane holds one key and 8 consecutive queries per k-step),
//    which makes P^T and dS^T ready-made A operands for dV += P^T dO and
//    dK += dS^T Q; dO and Q are read with the transposing LDS read. The
//    accumulators need one wave per SIMD; on unmasked tiles the two 32-query
//    halves of a tile are software-pipelined so that one half's exponentials
//    run between the other half's matrix products.
//  * bwd_dq_kernel: a work-group owns 128 queries (4 waves x 32) and walks the
//    key tiles, like the forward step: S^T = K Q^T and dP^T = V dO^T (Q and dO
//    fragments in registers), then dQ^T += K^T dS^T with K^T from the
//    transposing read.
// Tiles stream through double-buffered LDS via the DMA path; fully masked
// tiles are skipped from the positions (which increase), and only tiles
// across the diagonal (or ragged, or with ALiBi) are masked per element.
#include "tile_common.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr int D = 128;
constexpr int CPR = 16;             // 16-byte chunks per row
constexpr int KK = D / 16;          // k-steps over d
constexpr int DT = D / 32;          // 32-wide d tiles
constexpr int TROWS = 64;           // rows per streamed tile
constexpr int SLOTS = TROWS * CPR;  // 16-byte slots per tile
constexpr int DMA_PER_WAVE = SLOTS / (4 * 64);

__device__ __forceinline__ float safe_lse2(float lse) {
  // exp2(x - lse2) must give 0 for a row that saw no key (lse = -inf).
  return lse == -INFINITY ? INFINITY : lse * RA_LOG2E;
}

// Byte offsets (within a full tile) of this lane's DMA slots.
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[DMA_PER_WAVE], int wave, int lane) {
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int p = (wave * DMA_PER_WAVE + i) * 64 + lane;
    const int r = p / CPR, ph = p % CPR;
    off[i] = (uint32_t)(r * D + 8 * (ph ^ tile_swz(r))) * 2;
  }
}

// Copy rows [row0, row0 + 64) of a [L, 128] bf16 matrix into a swizzled LDS
// tile; rows at or past L are clamped to L - 1 (the caller masks them).
__device__ __forceinline__ void dma_tile(uint4* tile, const uint16_t* base, int row0, int L, int wave,
                                         int lane, const uint32_t (&off)[DMA_PER_WAVE]) {
  const char* t = reinterpret_cast<const char*>(base + (int64_t)row0 * D);
  if (row0 + TROWS <= L) {
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) dma16(t + off[i], &tile[(wave * DMA_PER_WAVE + i) * 64]);
  } else {
    const int last = L - 1 - row0;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int bs = (wave * DMA_PER_WAVE + i) * 64, p = bs + lane, r = p / CPR, ph = p % CPR;
      dma16(t + (uint32_t)(min(r, last) * D + 8 * (ph ^ tile_swz(r))) * 2, &tile[bs]);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

template <bool ALIBI>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a, int n_ktiles) {
  __shared__ uint4 Qs[2][SLOTS];
  __shared__ uint4 Os[2][SLOTS];  // dO
  __shared__ __align__(16) float lse_s[2][TROWS];
  __shared__ __align__(16) float del_s[2][TROWS];
  __shared__ __align__(16) int qp_s[2][TROWS];

  const int Lq = a.len_q, Lkv = a.len_kv;
  const int g = a.heads_q / a.heads_kv;
  const int bh = blockIdx.x / n_ktiles;  // (batch, kv head)
  const int kt = blockIdx.x - bh * n_ktiles;
  const int b = bh / a.heads_kv, hk = bh - b * a.heads_kv;

  const int tid = threadIdx.x;
  const int wave = uniform_i(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int k0 = kt * 128, kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;
  const bool key_ok = key < Lkv;
  const bool wave_active = kw0 < Lkv;
  const bool causal = a.causal != 0;
  const float c = a.scale * RA_LOG2E;

  const int64_t khead = (int64_t)b * a.heads_kv + hk;
  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.k) + khead * Lkv * D, (int64_t)Lkv * D * 2);
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.v) + khead * Lkv * D, (int64_t)Lkv * D * 2);

  // K and V fragments: B operands of S = Q K^T and dP = dO V^T (lane = key).
  uint4 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kf[kk] = buf_load16(rk, (uint32_t)(key * D + 16 * kk + 8 * hf) * 2);
    vf[kk] = buf_load16(rv, (uint32_t)(key * D + 16 * kk + 8 * hf) * 2);
  }
  const int my_kpos = key_ok ? a.k_pos[key] : INT32_MAX;
  const int kmin_w = wave_active ? a.k_pos[kw0] : INT32_MAX;
  const int kmax_w = wave_active ? a.k_pos[min(kw0 + 31, Lkv - 1)] : INT32_MAX;
  const int kmin_wg = a.k_pos[k0];

  // First query that can see any key of the work-group (positions increase).
  int qstart = 0;
  if (causal) {
    int lo = 0, hi = Lq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.q_pos[mid] < kmin_wg) lo = mid + 1; else hi = mid;
    }
    qstart = lo;
  }
  const int qt0 = qstart / TROWS;
  const int nq = (Lq + TROWS - 1) / TROWS - qt0;
  const int n_items = nq > 0 ? g * nq : 0;

  ra_f32x16 dK[DT], dV[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dK[dt] = ra_f32x16{};
    dV[dt] = ra_f32x16{};
  }

  if (n_items > 0) {
    uint32_t off[DMA_PER_WAVE];
    dma_offsets(off, wave, lane);
    auto item_head = [&](int it) { return hk * g + it / nq; };
    auto item_q0 = [&](int it) { return (qt0 + it % nq) * TROWS; };
    auto load_item = [&](int buf, int it) {
      const int hq = item_head(it), q0 = item_q0(it);
      const int64_t qhead = (int64_t)b * a.heads_q + hq;
      dma_tile(Qs[buf], static_cast<const uint16_t*>(a.q) + qhead * Lq * D, q0, Lq, wave, lane, off);
      dma_tile(Os[buf], static_cast<const uint16_t*>(a.d_o) + qhead * Lq * D, q0, Lq, wave, lane, off);
    };
    struct RowVals { float lse, del; int qp; };
    auto load_rows = [&](int it) {
      RowVals r{0.f, 0.f, 0};
      if (tid < TROWS) {
        const int hq = item_head(it), q = min(item_q0(it) + tid, Lq - 1);
        const int64_t row = ((int64_t)b * a.heads_q + hq) * Lq + q;
        r.lse = a.lse[row];  // converted when stored: no use before the loop's end
        r.del = a.delta[row];
        r.qp = a.q_pos[q];
      }
      return r;
    };
    auto store_rows = [&](int buf, const RowVals& r) {
      if (tid < TROWS) {
        lse_s[buf][tid] = safe_lse2(r.lse);
        del_s[buf][tid] = r.del;
        qp_s[buf][tid] = r.qp;
      }
    };

    // An item with masked elements (across the diagonal, ragged, or ALiBi):
    // one 32-query block after the other, masked per element.
    auto masked_item = [&](int buf, int q0, int hq) {
      const float sl2 = ALIBI ? a.slopes[hq] * RA_LOG2E : 0.0f;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        ra_f32x16 S = ra_f32x16{}, dP = ra_f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          S = ra_mfma32(tile_row_frag(Qs[buf], 32 * qb, kk, lane), kf[kk], S);
          dP = ra_mfma32(tile_row_frag(Os[buf], 32 * qb, kk, lane), vf[kk], dP);
        }
        // Lane element e: key `key`, query row 32*qb + 16*(e/8) + 8*hf + e%8.
        uint32_t Pw[8], Dw[8];
#pragma unroll
        for (int e8 = 0; e8 < 2; ++e8) {
          const int r0 = 32 * qb + 16 * e8 + 8 * hf;
          const float4 l0 = *reinterpret_cast<const float4*>(&lse_s[buf][r0]);
          const float4 l1 = *reinterpret_cast<const float4*>(&lse_s[buf][r0 + 4]);
          const float4 d0 = *reinterpret_cast<const float4*>(&del_s[buf][r0]);
          const float4 d1 = *reinterpret_cast<const float4*>(&del_s[buf][r0 + 4]);
          const int4 p0 = *reinterpret_cast<const int4*>(&qp_s[buf][r0]);
          const int4 p1 = *reinterpret_cast<const int4*>(&qp_s[buf][r0 + 4]);
          const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
          const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
          const int qv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float x = fmaf(S[8 * e8 + i], c, -lv[i]);
            if (ALIBI) x = fmaf(-sl2, (float)abs(qv[i] - my_kpos), x);
            const bool vis = (q0 + r0 + i < Lq) && key_ok && (!causal || my_kpos <= qv[i]);
            p[i] = vis ? __builtin_amdgcn_exp2f(x) : 0.0f;
          }
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            Pw[4 * e8 + i / 2] = ra_pack_bf16(p[i], p[i + 1]);
            Dw[4 * e8 + i / 2] =
                ra_pack_bf16(p[i] * (dP[8 * e8 + i] - dv[i]), p[i + 1] * (dP[8 * e8 + i + 1] - dv[i + 1]));
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 pa = make_uint4(Pw[4 * ks], Pw[4 * ks + 1], Pw[4 * ks + 2], Pw[4 * ks + 3]);
          const uint4 da = make_uint4(Dw[4 * ks], Dw[4 * ks + 1], Dw[4 * ks + 2], Dw[4 * ks + 3]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            dV[dt] = ra_mfma32(pa, tile_col_frag(Os[buf], 32 * qb + 16 * ks, 32 * dt, lane), dV[dt]);
            dK[dt] = ra_mfma32(da, tile_col_frag(Qs[buf], 32 * qb + 16 * ks, 32 * dt, lane), dK[dt]);
          }
        }
      }
    };

    // Per-lane parts of the fragment addresses. A row fragment of rows
    // r0 + perm_row(lane%32), k-step kk sits at byte r0*256 + (kk/4)*128 +
    // rofs[kk%4]; a column fragment (tile_col_frag) of rows r0, columns 32*dt
    // at r0*256 + (dt/2)*128 + cofs[half][dt%2] (the swizzle of a row depends
    // only on its offset inside a 16-row group, so r0 and the high column bit
    // add as constants).
    int rofs[4], cofs[2][2];
    {
      const int pr = perm_row(l32), g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
      for (int m = 0; m < 4; ++m) rofs[m] = pr * 256 + ((2 * m + hf) ^ tile_swz(pr)) * 16;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int rl = 8 * hf + 4 * half + (j >> 2), x = 2 * g + ((j & 3) >> 1);
          cofs[half][db] = rl * 256 + ((4 * db + x) ^ tile_swz(rl)) * 16 + 8 * (j & 1);
        }
    }
    auto row_frag = [&](const uint4* tile, int r0, int kk) {
      return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + r0 * 256 + (kk >> 2) * 128 +
                                             rofs[kk & 3]);
    };
    auto col_frag = [&](const uint4* tile, int r0, int dt) {
      const char* t = reinterpret_cast<const char*>(tile) + r0 * 256 + (dt >> 1) * 128;
      const uint2 a0 = lds_tr4(t + cofs[0][dt & 1]);
      const uint2 a1 = lds_tr4(t + cofs[1][dt & 1]);
      return make_uint4(a0.x, a0.y, a1.x, a1.y);
    };
    // An item every (query, key) pair of which is visible: no masks. With
    // one wave per SIMD the overlap of matrix and vector work has to come
    // from within the wave, so the code runs as
    //   S, dP (block 0) | S, dP (block 1), P and dS of block 0 in between
    //   | dV, dK (block 0), P and dS of block 1 in between | dV, dK (block 1)
    // with a scheduling fence after every step, and fragments are read a few
    // steps ahead of their products.
    auto fast_item = [&](int buf) {
      auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
      ra_f32x16 S[2], dP[2];
      uint32_t Pw[2][8], Dw[2][8];
      float lv[16], dv[16];  // lse, delta of the lane's 16 rows of one block
      auto load_lsedel = [&](int qb) {
#pragma unroll
        for (int e8 = 0; e8 < 2; ++e8) {
          const int r0 = 32 * qb + 16 * e8 + 8 * hf;
          const float4 l0 = *reinterpret_cast<const float4*>(&lse_s[buf][r0]);
          const float4 l1 = *reinterpret_cast<const float4*>(&lse_s[buf][r0 + 4]);
          const float4 d0 = *reinterpret_cast<const float4*>(&del_s[buf][r0]);
          const float4 d1 = *reinterpret_cast<const float4*>(&del_s[buf][r0 + 4]);
          lv[8 * e8 + 0] = l0.x; lv[8 * e8 + 1] = l0.y; lv[8 * e8 + 2] = l0.z; lv[8 * e8 + 3] = l0.w;
          lv[8 * e8 + 4] = l1.x; lv[8 * e8 + 5] = l1.y; lv[8 * e8 + 6] = l1.z; lv[8 * e8 + 7] = l1.w;
          dv[8 * e8 + 0] = d0.x; dv[8 * e8 + 1] = d0.y; dv[8 * e8 + 2] = d0.z; dv[8 * e8 + 3] = d0.w;
          dv[8 * e8 + 4] = d1.x; dv[8 * e8 + 5] = d1.y; dv[8 * e8 + 6] = d1.z; dv[8 * e8 + 7] = d1.w;
        }
      };
      // VALU work of block qb for elements 2*j, 2*j + 1: P, dS, both packed.
      auto valu = [&](int qb, int j) {
        const int e = 2 * j;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S[qb][e], c, -lv[e]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S[qb][e + 1], c, -lv[e + 1]));
        Pw[qb][j] = ra_pack_bf16(p0, p1);
        Dw[qb][j] = ra_pack_bf16(p0 * (dP[qb][e] - dv[e]), p1 * (dP[qb][e + 1] - dv[e + 1]));
      };
      // S, dP of block qb; row fragments read LA k-steps ahead; extra(kk)
      // runs between the k-steps.
      constexpr int LA = 3;
      auto sdp = [&](int qb, auto extra) {
        uint4 qa[LA + 1], oa[LA + 1];
#pragma unroll
        for (int kk = 0; kk < LA; ++kk) {
          qa[kk] = row_frag(Qs[buf], 32 * qb, kk);
          oa[kk] = row_frag(Os[buf], 32 * qb, kk);
        }
        S[qb] = ra_f32x16{};
        dP[qb] = ra_f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + LA < KK) {
            qa[(kk + LA) % (LA + 1)] = row_frag(Qs[buf], 32 * qb, kk + LA);
            oa[(kk + LA) % (LA + 1)] = row_frag(Os[buf], 32 * qb, kk + LA);
          }
          S[qb] = ra_mfma32(qa[kk % (LA + 1)], kf[kk], S[qb]);
          dP[qb] = ra_mfma32(oa[kk % (LA + 1)], vf[kk], dP[qb]);
          extra(kk);
          fence();
        }
      };
      // dV, dK of block qb; column fragments read one step ahead.
      auto dvdk = [&](int qb, bool with_valu) {
        uint4 ob[2], qbf[2];
        ob[0] = col_frag(Os[buf], 32 * qb, 0);
        qbf[0] = col_frag(Qs[buf], 32 * qb, 0);
#pragma unroll
        for (int st = 0; st < 2 * DT; ++st) {  // st = ks * DT + dt
          const int ks = st / DT, dt = st % DT;
          if (st + 1 < 2 * DT) {
            const int ks1 = (st + 1) / DT, dt1 = (st + 1) % DT;
            ob[(st + 1) & 1] = col_frag(Os[buf], 32 * qb + 16 * ks1, dt1);
            qbf[(st + 1) & 1] = col_frag(Qs[buf], 32 * qb + 16 * ks1, dt1);
          }
          const uint4 pa = make_uint4(Pw[qb][4 * ks], Pw[qb][4 * ks + 1], Pw[qb][4 * ks + 2], Pw[qb][4 * ks + 3]);
          const uint4 da = make_uint4(Dw[qb][4 * ks], Dw[qb][4 * ks + 1], Dw[qb][4 * ks + 2], Dw[qb][4 * ks + 3]);
          dV[dt] = ra_mfma32(pa, ob[st & 1], dV[dt]);
          dK[dt] = ra_mfma32(da, qbf[st & 1], dK[dt]);
          if (with_valu) valu(1, st);
          fence();
        }
      };
      load_lsedel(0);
      sdp(0, [](int) {});
      sdp(1, [&](int kk) { valu(0, kk); });
      load_lsedel(1);
      dvdk(0, true);
      dvdk(1, false);
    };
    load_item(0, 0);
    store_rows(0, load_rows(0));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

#pragma clang loop unroll(disable)
    for (int it = 0;; ++it) {
      const int buf = it & 1;
      const bool have_next = it + 1 < n_items;
      RowVals nxt{0.f, 0.f, 0};
      if (have_next) {
        load_item(buf ^ 1, it + 1);
        nxt = load_rows(it + 1);
      }
      const int hq = item_head(it), q0 = item_q0(it);
      // Positions of the item's first and last query row, from the LDS copy
      // (kept off the vector-memory counter that the tile copies use).
      const int qfirst = uniform_i(qp_s[buf][0]);
      const int qlast = uniform_i(qp_s[buf][TROWS - 1]);
      if (wave_active && !(causal && qlast < kmin_w)) {
        const bool diag = (q0 + TROWS > Lq) || (causal && qfirst < kmax_w) || ALIBI;
        if (!diag) {
          fast_item(buf);
        } else {
          masked_item(buf, q0, hq);
        }
      }
      if (!have_next) break;
      store_rows(buf ^ 1, nxt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // Accumulate into dk_blk / dv_blk: element (dt, e) is key kw0 + 8*(e/4) +
  // 4*hf + e%4, dim 32*dt + l32.
  if (!wave_active) return;
  float* dkh = a.dk + khead * Lkv * D;
  float* dvh = a.dv + khead * Lkv * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = kw0 + 8 * (e >> 2) + 4 * hf + (e & 3);
      if (kr < Lkv) {
        const int64_t idx = (int64_t)kr * D + 32 * dt + l32;
        dkh[idx] += a.scale * dK[dt][e];
        dvh[idx] += dV[dt][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

template <bool ALIBI>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a, int n_qtiles) {
  __shared__ uint4 Ks[2][SLOTS];
  __shared__ uint4 Vs[2][SLOTS];
  __shared__ __align__(16) int kp[2][TROWS];

  const int Lq = a.len_q, Lkv = a.len_kv;
  const int bh = blockIdx.x / n_qtiles;
  const int qt = n_qtiles - 1 - (blockIdx.x - bh * n_qtiles);  // heaviest first under causal
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);

  const int tid = threadIdx.x;
  const int wave = uniform_i(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int q0 = qt * 128, q0w = q0 + 32 * wave;
  const int row = q0w + l32;
  const bool row_ok = row < Lq;
  const bool wave_active = q0w < Lq;
  const bool causal = a.causal != 0;
  const float c = a.scale * RA_LOG2E;

  const int64_t qhead = (int64_t)b * a.heads_q + h;
  const int64_t khead = (int64_t)b * a.heads_kv + hk;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + khead * Lkv * D;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + khead * Lkv * D;
  const auto rq = make_rsrc(static_cast<const uint16_t*>(a.q) + qhead * Lq * D, (int64_t)Lq * D * 2);
  const auto rdo = make_rsrc(static_cast<const uint16_t*>(a.d_o) + qhead * Lq * D, (int64_t)Lq * D * 2);
  const int* kpos = a.k_pos;

  const int qmax_wg = a.q_pos[min(q0 + 127, Lq - 1)];
  auto tile_live = [&](int kv0) { return kv0 < Lkv && (!causal || kpos[kv0] <= qmax_wg); };
  if (!tile_live(0)) return;

  const int qmin_w = wave_active ? a.q_pos[q0w] : INT32_MAX;
  const int qmax_w = wave_active ? a.q_pos[min(q0w + 31, Lq - 1)] : INT32_MIN;
  const int my_pos = row_ok ? a.q_pos[row] : INT32_MAX;
  const float my_lse2 = row_ok ? safe_lse2(a.lse[qhead * Lq + row]) : INFINITY;
  const float my_del = row_ok ? a.delta[qhead * Lq + row] : 0.0f;
  const float sl2 = ALIBI ? a.slopes[h] * RA_LOG2E : 0.0f;

  // Q and dO fragments: B operands of S^T = K Q^T and dP^T = V dO^T.
  uint4 qf[KK], of[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = buf_load16(rq, (uint32_t)(row * D + 16 * kk + 8 * hf) * 2);
    of[kk] = buf_load16(rdo, (uint32_t)(row * D + 16 * kk + 8 * hf) * 2);
  }
  ra_f32x16 dQ[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dQ[dt] = ra_f32x16{};
  bool touched = false;

  uint32_t off[DMA_PER_WAVE];
  dma_offsets(off, wave, lane);
  auto load_kp = [&](int kv0) { return tid < TROWS ? kpos[min(kv0 + tid, Lkv - 1)] : 0; };

  dma_tile(Ks[0], kh, 0, Lkv, wave, lane, off);
  dma_tile(Vs[0], vh, 0, Lkv, wave, lane, off);
  if (tid < TROWS) kp[0][tid] = load_kp(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

#pragma clang loop unroll(disable)
  for (int kv0 = 0, t = 0;; kv0 += TROWS, ++t) {
    const int buf = t & 1;
    // The next tile is copied whenever it exists; whether any query of the
    // work-group sees it is decided once its positions are in LDS.
    const bool have_next = kv0 + TROWS < Lkv;
    int kp_next = 0;
    if (have_next) {
      dma_tile(Ks[buf ^ 1], kh, kv0 + TROWS, Lkv, wave, lane, off);
      dma_tile(Vs[buf ^ 1], vh, kv0 + TROWS, Lkv, wave, lane, off);
      kp_next = load_kp(kv0 + TROWS);
    }
    const int kfirst = uniform_i(kp[buf][0]);
    const int klast = uniform_i(kp[buf][TROWS - 1]);
    if (wave_active && !(causal && kfirst > qmax_w)) {
      touched = true;
      const bool diag = (kv0 + TROWS > Lkv) || (causal && klast > qmin_w) || ALIBI;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        ra_f32x16 S = ra_f32x16{}, dP = ra_f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          S = ra_mfma32(tile_row_frag(Ks[buf], 32 * sb, kk, lane), qf[kk], S);
          dP = ra_mfma32(tile_row_frag(Vs[buf], 32 * sb, kk, lane), of[kk], dP);
        }
        // Lane element e: query `row`, key 32*sb + 16*(e/8) + 8*hf + e%8.
        uint32_t Dw[8];
#pragma unroll
        for (int e8 = 0; e8 < 2; ++e8) {
          const int j0 = 32 * sb + 16 * e8 + 8 * hf;
          float ds[8];
          if (diag) {
            const int4 p0 = *reinterpret_cast<const int4*>(&kp[buf][j0]);
            const int4 p1 = *reinterpret_cast<const int4*>(&kp[buf][j0 + 4]);
            const int kv8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              float x = fmaf(S[8 * e8 + i], c, -my_lse2);
              if (ALIBI) x = fmaf(-sl2, (float)abs(my_pos - kv8[i]), x);
              const bool vis = (kv0 + j0 + i < Lkv) && (!causal || kv8[i] <= my_pos);
              const float p = vis ? __builtin_amdgcn_exp2f(x) : 0.0f;
              ds[i] = p * (dP[8 * e8 + i] - my_del);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(S[8 * e8 + i], c, -my_lse2));
              ds[i] = p * (dP[8 * e8 + i] - my_del);
            }
          }
#pragma unroll
          for (int i = 0; i < 8; i += 2) Dw[4 * e8 + i / 2] = ra_pack_bf16(ds[i], ds[i + 1]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 db = make_uint4(Dw[4 * ks], Dw[4 * ks + 1], Dw[4 * ks + 2], Dw[4 * ks + 3]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            dQ[dt] = ra_mfma32(tile_col_frag(Ks[buf], 32 * sb + 16 * ks, 32 * dt, lane), db, dQ[dt]);
        }
      }
    }
    if (!have_next) break;
    if (tid < TROWS) kp[buf ^ 1][tid] = kp_next;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (causal && uniform_i(kp[buf ^ 1][0]) > qmax_wg) break;  // keys past the last query
  }

  if (!touched || !row_ok) return;
  // dq_acc += scale * dQ; element (dt, e) of this lane is dim 32*dt +
  // 8*(e/4) + 4*hf + e%4 of query `row`.
  float* dqr = a.dq + (qhead * Lq + row) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      float4* p = reinterpret_cast<float4*>(dqr + 32 * dt + 8 * a4 + 4 * hf);
      float4 v = *p;
      v.x += a.scale * dQ[dt][4 * a4 + 0];
      v.y += a.scale * dQ[dt][4 * a4 + 1];
      v.z += a.scale * dQ[dt][4 * a4 + 2];
      v.w += a.scale * dQ[dt][4 * a4 + 3];
      *p = v;
    }
  }
}

template <bool ALIBI>
hipError_t launch_both(const BwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.len_q + 127) / 128;
  const int n_ktiles = (a.len_kv + 127) / 128;
  const int64_t grid_q = (int64_t)n_qtiles * a.batch * a.heads_q;
  const int64_t grid_k = (int64_t)n_ktiles * a.batch * a.heads_kv;
  if (grid_q > INT32_MAX || grid_k > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_kernel<ALIBI>), dim3((unsigned)grid_q), dim3(kThreads), 0, stream, a, n_qtiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<ALIBI>), dim3((unsigned)grid_k), dim3(kThreads), 0, stream, a, n_ktiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  return a.slopes ? launch_both<true>(a, stream) : launch_both<false>(a, stream);
}

}  // namespace ra
