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
//  * bwd_dkdv_kernel: a work-group owns 128 keys (4 blocks of 32) of one K/V
//    head and walks every query head of its group and every 64-query tile that
//    sees those keys. Each key block has two waves on one SIMD, split by
//    output: the dV wave holds the K fragments and the dV accumulator and
//    computes S = Q K^T, P and dV += P^T dO; the dK wave holds the V fragments
//    and the dK accumulator and computes dP = dO V^T, reads P from LDS, and
//    forms dS and dK += dS^T Q. Per tile: S | dP, then (barrier) dV | dS, dK;
//    the two waves' matrix and vector work overlap on their SIMD, and the dK
//    waves issue the next tile's copies in the slack of the first half. S and
//    dP run with the query rows as the MFMA A operand (rows permuted so that
//    each lane holds one key and 8 consecutive queries per k-step), which
//    makes P^T and dS^T ready-made A operands of the next products; dO and Q
//    are read with the transposing LDS read.
//  * bwd_dq_kernel: a work-group takes 128 queries (4 waves x 32) at a time and
//    walks the key tiles, like the forward step: S^T = K Q^T and dP^T = V dO^T
//    (Q and dO fragments in registers), then dQ^T += K^T dS^T with K^T from the
//    transposing read. The launch is persistent (two work-groups per CU at
//    most), with each XCD taking its heads one at a time, as in the forward.
// Tiles stream through double-buffered LDS via the DMA path; fully masked
// tiles are skipped from the positions (which increase), and only tiles
// across the diagonal (or ragged, or with ALiBi) are masked per element.
#include <type_traits>

#include "tile_common.h"

namespace ra {
namespace {

constexpr int kThreads = 256;       // dQ work-group: 4 waves x 32 queries
constexpr int kThreadsKV = 512;     // dK/dV work-group: 4 key blocks x (dV wave, dK wave)
constexpr int D = 128;
constexpr int CPR = 16;             // 16-byte chunks per row
constexpr int KK = D / 16;          // k-steps over d
constexpr int DT = D / 32;          // 32-wide d tiles
constexpr int TROWS = kTileRows;    // rows per streamed tile (64)
constexpr int SLOTS = TROWS * CPR;  // 16-byte slots per tile

__device__ __forceinline__ float safe_lse2(float lse) {
  // exp2(x - lse2) must give 0 for a row that saw no key (lse = -inf).
  return lse == -INFINITY ? INFINITY : lse * RA_LOG2E;
}

// A 64-row tile is copied by NW waves, DPW = SLOTS / (64 * NW) 16-byte slots
// per lane, in the layout of tile_slot.
template <int NW>
struct TileCopy {
  static constexpr int DPW = SLOTS / (64 * NW);
  uint32_t off[DPW];  // byte offsets of this lane's slots within a full tile
  __device__ __forceinline__ TileCopy(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      int r;
      const int ch = tile_slot_chunk((wave * DPW + i) * 64 + lane, &r);
      off[i] = (uint32_t)(r * D + 8 * ch) * 2;
    }
  }
  // Copy rows [row0, row0 + 64) of a [L, 128] bf16 matrix (0 <= row0 < L);
  // rows at or past L are clamped to L - 1 (the caller masks them).
  __device__ __forceinline__ void copy(uint4* tile, const uint16_t* base, int row0, int L, int wave,
                                       int lane) const {
    const char* t = reinterpret_cast<const char*>(base + (int64_t)row0 * D);
    if (row0 + TROWS <= L) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) dma16(t + off[i], &tile[(wave * DPW + i) * 64]);
    } else {
      const int last = L - 1 - row0;
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int bs = (wave * DPW + i) * 64;
        int r;
        const int ch = tile_slot_chunk(bs + lane, &r);
        dma16(t + (uint32_t)(min(r, last) * D + 8 * ch) * 2, &tile[bs]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

template <bool ALIBI>
__global__ __launch_bounds__(kThreadsKV, 1) void bwd_dkdv_kernel(BwdArgs a, int n_ktiles) {
  __shared__ uint4 Qs[2][SLOTS];
  __shared__ uint4 Os[2][SLOTS];  // dO
  __shared__ __align__(16) float lse_s[2][TROWS];
  __shared__ __align__(16) float del_s[2][TROWS];  // -delta per query row
  __shared__ __align__(16) int qp_s[2][TROWS];
  // Under ALiBi: -(lse * log2 e + slope * log2 e * (q_pos - first query of
  // the item)) / (scale * log2 e) per query row, the start value of S on the
  // items a key block sees in full.
  __shared__ __align__(16) float lsec_s[ALIBI ? 2 : 1][TROWS];
  // P of the current tile, handed from each key block's dV wave to its dK
  // wave: [key block][query half][element quad][lane], 4 floats each.
  __shared__ float4 Px[4][2][4][64];

  const int Lq = a.len_q, Lkv = a.len_kv;
  const int g = a.heads_q / a.heads_kv;
  // Key tiles in order of decreasing work across all heads (tile 0 sees the
  // most queries under the causal mask), so the lightest work-groups come
  // last; head bh then always lands on XCD bh % 8.
  const int n_bh = (int)(gridDim.x / (unsigned)n_ktiles);
  const int kt = blockIdx.x / n_bh;
  const int bh = blockIdx.x - kt * n_bh;  // (batch, kv head)
  const int b = bh / a.heads_kv, hk = bh - b * a.heads_kv;

  const int tid = threadIdx.x;
  const int wave = uniform_i(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  // Waves kb and kb + 4 share a SIMD and key block kb: the first computes
  // S, P and dV, the second dP, dS and dK.
  const int kb = wave & 3;
  const bool dv_wave = wave < 4;
  const int k0 = kt * 128, kw0 = k0 + 32 * kb;
  const int key = kw0 + l32;
  const bool key_ok = key < Lkv;
  const bool wave_active = kw0 < Lkv;
  const bool causal = a.causal != 0;
  const float c = a.scale * RA_LOG2E;
  // The linear form of the ALiBi term divides by c: with c <= 0 every item
  // takes the per-element path (as in the forward step).
  const bool lin_ok = c > 0.0f;

  const int64_t khead = (int64_t)b * a.heads_kv + hk;
  // K fragments (B operand of S = Q K^T) for the dV wave, V fragments (B
  // operand of dP = dO V^T) for the dK wave; lane = key.
  const auto rkv = make_rsrc(static_cast<const uint16_t*>(dv_wave ? a.k : a.v) + khead * Lkv * D,
                             (int64_t)Lkv * D * 2);
  uint4 bf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) bf[kk] = buf_load16(rkv, (uint32_t)(key * D + 16 * kk + 8 * hf) * 2);
  const int my_kpos = key_ok ? a.k_pos[key] : INT32_MAX;
  const int kmin_w = wave_active ? a.k_pos[kw0] : INT32_MAX;
  const int kmax_w = wave_active ? a.k_pos[min(kw0 + 31, Lkv - 1)] : INT32_MAX;
  const int kmin_wg = a.k_pos[k0];

  // First query tile that can see a key of the work-group: the tiles before
  // it end below the work-group's first key (positions increase).
  int qt0 = 0;
  if (causal)
    qt0 = prefix_count((Lq + TROWS - 1) / TROWS, lane,
                       [&](int u) { return a.q_pos[min(u * TROWS + TROWS - 1, Lq - 1)] < kmin_wg; });
  const int nq = (Lq + TROWS - 1) / TROWS - qt0;
  const int n_items = nq > 0 ? g * nq : 0;

  ra_f32x16 acc[DT];  // dV (dV wave) or dK / scale (dK wave)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = ra_f32x16{};

  if (n_items > 0) {
    // The dK waves copy the tiles (in their slack at the end of the first
    // phase of the previous item); the dV waves copy nothing.
    const TileCopy<4> tc(kb, lane);
    auto item_head = [&](int it) { return hk * g + it / nq; };
    auto item_q0 = [&](int it) { return (qt0 + it % nq) * TROWS; };
    auto load_item = [&](int buf, int it) {
      const int hq = item_head(it), q0 = item_q0(it);
      const int64_t qhead = (int64_t)b * a.heads_q + hq;
      tc.copy(Qs[buf], static_cast<const uint16_t*>(a.q) + qhead * Lq * D, q0, Lq, kb, lane);
      tc.copy(Os[buf], static_cast<const uint16_t*>(a.d_o) + qhead * Lq * D, q0, Lq, kb, lane);
    };
    struct RowVals { float lse, del, sl2; int qp, qb; };
    auto load_rows = [&](int it) {
      RowVals r{0.f, 0.f, 0.f, 0, 0};
      if (tid < TROWS) {
        const int hq = item_head(it), q = min(item_q0(it) + tid, Lq - 1);
        const int64_t row = ((int64_t)b * a.heads_q + hq) * Lq + q;
        r.lse = a.lse[row];  // converted when stored: no use before the loop's end
        r.del = a.delta[row];
        r.qp = a.q_pos[q];
        if constexpr (ALIBI) {
          r.sl2 = a.slopes[hq] * RA_LOG2E;
          r.qb = a.q_pos[item_q0(it)];
        }
      }
      return r;
    };
    auto store_rows = [&](int buf, const RowVals& r) {
      if (tid < TROWS) {
        const float l2 = safe_lse2(r.lse);
        lse_s[buf][tid] = l2;
        del_s[buf][tid] = -r.del;  // the start value of dP
        qp_s[buf][tid] = r.qp;
        if constexpr (ALIBI) lsec_s[buf][tid] = lin_ok ? -(l2 + r.sl2 * (float)(r.qp - r.qb)) / c : 0.0f;
      }
    };

    // Per-lane parts of the fragment addresses (the rest folds into the
    // instructions' immediate offsets).
    const FragOffsets fo(lane);
    auto row_frag = [&](const uint4* tile, int r0, int kk) { return tile_row_frag(tile, r0, kk, fo); };
    auto col_frag = [&](const uint4* tile, int r0, int dt) { return tile_col_frag(tile, r0, dt, fo); };
    // One 32-query block's product A(rows) x bf^T: S (dV wave) or dP (dK wave).
    constexpr int LA = 3;
    auto row_product = [&](const uint4* tile, int qb, ra_f32x16 r) {
      uint4 fr[LA + 1];
#pragma unroll
      for (int kk = 0; kk < LA; ++kk) fr[kk] = row_frag(tile, 32 * qb, kk);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + LA < KK) fr[(kk + LA) % (LA + 1)] = row_frag(tile, 32 * qb, kk + LA);
        r = ra_mfma32(fr[kk % (LA + 1)], bf[kk], r);
      }
      return r;
    };
    // acc += W^T T for one 32-query block: W (8 packed bf16 pairs per lane)
    // is P^T or dS^T, T the dO or Q tile read by column.
    auto col_product = [&](const uint4* tile, int qb, const uint32_t (&W)[8]) {
      uint4 cf[2];
      cf[0] = col_frag(tile, 32 * qb, 0);
#pragma unroll
      for (int st = 0; st < 2 * DT; ++st) {  // st = ks * DT + dt
        const int ks = st / DT, dt = st % DT;
        if (st + 1 < 2 * DT) cf[(st + 1) & 1] = col_frag(tile, 32 * qb + 16 * ((st + 1) / DT), (st + 1) % DT);
        const uint4 w = make_uint4(W[4 * ks], W[4 * ks + 1], W[4 * ks + 2], W[4 * ks + 3]);
        acc[dt] = ra_mfma32(w, cf[st & 1], acc[dt]);
      }
    };

    if (!dv_wave) load_item(0, 0);
    store_rows(0, load_rows(0));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

#pragma clang loop unroll(disable)
    for (int it = 0;; ++it) {
      const int buf = it & 1;
      const bool have_next = it + 1 < n_items;
      RowVals nxt{0.f, 0.f, 0};
      if (have_next) nxt = load_rows(it + 1);
      const int hq = item_head(it), q0 = item_q0(it);
      // Positions of the item's first and last query row, from the LDS copy
      // (kept off the vector-memory counter that the tile copies use).
      const int qfirst = uniform_i(qp_s[buf][0]);
      const int qlast = uniform_i(qp_s[buf][TROWS - 1]);
      const bool active = wave_active && !(causal && qlast < kmin_w);
      // Under the causal mask the ALiBi term of an item the key block sees
      // in full is -slope * (q_pos - k_pos): its row part (with the LSE) is
      // S's start value and its key part the per-lane offset; only ALiBi
      // without the causal mask needs the per-element form everywhere.
      const bool masked = (q0 + TROWS > Lq) || (causal && qfirst < kmax_w) || (ALIBI && !(causal && lin_ok));
      // Lane element e of a block: key `key`, query row 32*qb + 16*(e/8) + 8*hf + e%8.
      // Carried across the barrier in the same registers: dP = dO V^T of both
      // blocks (dK wave), or P^T packed to bf16 pairs (dV wave, in hold[qb][0..7]).
      ra_f32x16 hold[2];
      uint32_t W[2][8];
      // The wave with vector work in a half has the longer path: it gets
      // issue priority over its partner for that half.
      if (dv_wave) __builtin_amdgcn_s_setprio(1);
      if (active) {
        if (dv_wave) {
          const float sl2 = ALIBI ? a.slopes[hq] * RA_LOG2E : 0.0f;
          // The mask test is hoisted out of the block loop, so each variant is
          // one straight-line stretch in which the second block's products can
          // issue among the first block's exponentials.
          auto s_and_p = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const float kc = sl2 * (float)(my_kpos - qfirst);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              ra_f32x16 S0 = ra_f32x16{};
              if constexpr (ALIBI && !MASKED) {
                const float4* lv4 = reinterpret_cast<const float4*>(&lsec_s[buf][32 * qb + 8 * hf]);
                const float4 x0 = lv4[0], x1 = lv4[1], x2 = lv4[4], x3 = lv4[5];
                S0 = ra_f32x16{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                               x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
              }
              const ra_f32x16 S = row_product(Qs[buf], qb, S0);
              float p[16];
#pragma unroll
              for (int e8 = 0; e8 < 2; ++e8) {
                const int r0 = 32 * qb + 16 * e8 + 8 * hf;
                const float4 l0 = *reinterpret_cast<const float4*>(&lse_s[buf][r0]);
                const float4 l1 = *reinterpret_cast<const float4*>(&lse_s[buf][r0 + 4]);
                const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                if constexpr (MASKED) {
                  const int4 p0 = *reinterpret_cast<const int4*>(&qp_s[buf][r0]);
                  const int4 p1 = *reinterpret_cast<const int4*>(&qp_s[buf][r0 + 4]);
                  const int qv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
                  for (int i = 0; i < 8; ++i) {
                    float x = fmaf(S[8 * e8 + i], c, -lv[i]);
                    if (ALIBI) x = fmaf(-sl2, (float)abs(qv[i] - my_kpos), x);
                    // bitwise, not short-circuit: no branch per element
                    const bool vis = (q0 + r0 + i < Lq) & key_ok & (!causal | (my_kpos <= qv[i]));
                    p[8 * e8 + i] = vis ? __builtin_amdgcn_exp2f(x) : 0.0f;
                  }
                } else if constexpr (ALIBI) {
#pragma unroll
                  for (int i = 0; i < 8; ++i) p[8 * e8 + i] = __builtin_amdgcn_exp2f(fmaf(S[8 * e8 + i], c, kc));
                } else {
#pragma unroll
                  for (int i = 0; i < 8; ++i) p[8 * e8 + i] = __builtin_amdgcn_exp2f(fmaf(S[8 * e8 + i], c, -lv[i]));
                }
              }
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                Px[kb][qb][q4][lane] = make_float4(p[4 * q4], p[4 * q4 + 1], p[4 * q4 + 2], p[4 * q4 + 3]);
#pragma unroll
              for (int i = 0; i < 8; ++i) hold[qb][i] = __uint_as_float(ra_pack_bf16(p[2 * i], p[2 * i + 1]));
            }
          };
          if (masked) s_and_p(std::true_type{});
          else s_and_p(std::false_type{});
        } else {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            // dP starts from -delta of its query rows, so that dP - delta
            // comes out of the product.
            const float4* d4 = reinterpret_cast<const float4*>(&del_s[buf][32 * qb + 8 * hf]);
            const float4 x0 = d4[0], x1 = d4[1], x2 = d4[4], x3 = d4[5];
            const ra_f32x16 nd = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                  x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
            hold[qb] = row_product(Os[buf], qb, nd);
          }
        }
      }
      if (!dv_wave && have_next) load_item(buf ^ 1, it + 1);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();  // P of this tile is in Px
      if (!dv_wave) __builtin_amdgcn_s_setprio(1);
      if (active) {
        // W is P^T (dV wave) or dS^T (dK wave); both waves then run the same
        // products from one call site, so the accumulator keeps one set of
        // registers (two call sites made the compiler copy it out and back
        // on every tile).
        if (dv_wave) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 8; ++i) W[qb][i] = __float_as_uint(hold[qb][i]);
        } else {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int e8 = 0; e8 < 2; ++e8) {
              const float4 pa = Px[kb][qb][2 * e8][lane], pb = Px[kb][qb][2 * e8 + 1][lane];
              const float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
              for (int i = 0; i < 8; i += 2)
                W[qb][4 * e8 + i / 2] = ra_pack_bf16(p[i] * hold[qb][8 * e8 + i],
                                                     p[i + 1] * hold[qb][8 * e8 + i + 1]);
            }
          }
        }
        const uint4* T = dv_wave ? Os[buf] : Qs[buf];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) col_product(T, qb, W[qb]);
      }
      __builtin_amdgcn_s_setprio(0);
      if (!have_next) break;
      store_rows(buf ^ 1, nxt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // Accumulate into dv_blk (dV wave) or dk_blk (dK wave): element (dt, e) is
  // key kw0 + 8*(e/4) + 4*hf + e%4, dim 32*dt + l32. Through a buffer
  // resource that starts at the wave's first key and ends at the chunk's
  // end, so that rows past it read zeros and drop their stores with no
  // branch; all 64 loads are issued before the first sum, so the wave waits
  // for memory once rather than once per element.
  if (!wave_active) return;
  const auto rout = make_rsrc((dv_wave ? a.dv : a.dk) + (khead * Lkv + kw0) * D, (int64_t)(Lkv - kw0) * D * 4);
  const float f = dv_wave ? 1.0f : a.scale;
  auto out_off = [&](int dt, int e) { return (uint32_t)(((8 * (e >> 2) + 4 * hf + (e & 3)) * D + 32 * dt + l32) * 4); };
  float old[DT][16];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) old[dt][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rout, out_off(dt, e), 0, 0));
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(f, acc[dt][e], old[dt][e])), rout, out_off(dt, e), 0, 0);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

template <bool ALIBI>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a, int n_qtiles, int groups) {
  __shared__ uint4 Ks[2][SLOTS];
  __shared__ uint4 Vs[2][SLOTS];
  __shared__ __align__(16) int kp[2][TROWS];
  // Under ALiBi: slope * (k_pos - first key of the tile) / scale per key, the
  // start value of S on the tiles the wave sees in full.
  __shared__ __align__(16) float kbc[ALIBI ? 2 : 1][TROWS];

  const int BH = a.batch * a.heads_q;

  // One 128-query tile of one head; the work-group walks a list of them (see
  // the loop at the end).
  using CArgs = const __attribute__((address_space(4))) BwdArgs;
  auto run_task = [&](CArgs& a, const int tid, const int bh_in, const int qt_in) {
  // Uniform across the work-group; said so, so that addresses derived from them stay scalar.
  const int bh = uniform_i(bh_in), qt = uniform_i(qt_in);
  const int Lq = a.len_q, Lkv = a.len_kv;
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
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
  // The linear form of the ALiBi term divides by the scale: with c <= 0
  // every tile takes the per-element path (as in the forward step).
  const bool lin_ok = c > 0.0f;
  const float sl2 = ALIBI ? a.slopes[h] * RA_LOG2E : 0.0f;
  const float sl2c = (ALIBI && lin_ok) ? a.slopes[h] / a.scale : 0.0f;

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

  const TileCopy<4> tc(wave, lane);
  const FragOffsets fo(lane);
  auto load_kp = [&](int kv0) { return tid < TROWS ? kpos[min(kv0 + tid, Lkv - 1)] : 0; };

  auto store_kp = [&](int buf, int kv0, int kpv) {
    if (tid < TROWS) {
      kp[buf][tid] = kpv;
      if constexpr (ALIBI) kbc[buf][tid] = sl2c * (float)(kpv - kpos[kv0]);
    }
  };
  tc.copy(Ks[0], kh, 0, Lkv, wave, lane);
  tc.copy(Vs[0], vh, 0, Lkv, wave, lane);
  store_kp(0, 0, load_kp(0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One key tile; false when the walk ends. FULL: a tile that every row of
  // the work-group sees in full, whose body then has no mask test at all (a
  // per-tile test inside the block loop splits it into branches the
  // scheduler cannot interleave across).
  auto tile_step = [&](int kv0, int t, auto full_tag) -> bool {
    constexpr bool FULL = decltype(full_tag)::value;
    const int buf = t & 1;
    // The next tile is copied whenever it exists; whether any query of the
    // work-group sees it is decided once its positions are in LDS.
    const bool have_next = kv0 + TROWS < Lkv;
    int kp_next = 0;
    if (have_next) {
      tc.copy(Ks[buf ^ 1], kh, kv0 + TROWS, Lkv, wave, lane);
      tc.copy(Vs[buf ^ 1], vh, kv0 + TROWS, Lkv, wave, lane);
      kp_next = load_kp(kv0 + TROWS);
    }
    const int kfirst = uniform_i(kp[buf][0]);
    const int klast = uniform_i(kp[buf][TROWS - 1]);
    if (wave_active && !(causal && kfirst > qmax_w)) {
      touched = true;
      // Per-element masks only across the diagonal, on a ragged tile, or
      // for ALiBi without the causal mask. Under the causal mask the ALiBi
      // term of a tile the wave sees in full is -slope * (q_pos - k_pos): its
      // key part is S's start value and its row part joins the LSE offset.
      const bool diag =
          !FULL && ((kv0 + TROWS > Lkv) || (causal && klast > qmin_w) || (ALIBI && !(causal && lin_ok)));
      const float row_off = ALIBI ? -my_lse2 - sl2 * (float)(my_pos - kfirst) : -my_lse2;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        ra_f32x16 S = ra_f32x16{}, dP = ra_f32x16{};
        if constexpr (ALIBI) {
          if (!diag) {
            const float4* kv = reinterpret_cast<const float4*>(&kbc[buf][32 * sb + 8 * hf]);
            const float4 x0 = kv[0], x1 = kv[1], x2 = kv[4], x3 = kv[5];
            S = ra_f32x16{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                          x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
          }
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          S = ra_mfma32(tile_row_frag(Ks[buf], 32 * sb, kk, fo), qf[kk], S);
          dP = ra_mfma32(tile_row_frag(Vs[buf], 32 * sb, kk, fo), of[kk], dP);
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
              // bitwise, not short-circuit: no branch per element
              const bool vis = (kv0 + j0 + i < Lkv) & (!causal | (kv8[i] <= my_pos));
              const float p = vis ? __builtin_amdgcn_exp2f(x) : 0.0f;
              ds[i] = p * (dP[8 * e8 + i] - my_del);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(S[8 * e8 + i], c, row_off));
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
            dQ[dt] = ra_mfma32(tile_col_frag(Ks[buf], 32 * sb + 16 * ks, dt, fo), db, dQ[dt]);
        }
      }
    }
    if (!have_next) return false;
    store_kp(buf ^ 1, kv0 + TROWS, kp_next);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // keys past the last query end the walk
    return !(causal && uniform_i(kp[buf ^ 1][0]) > qmax_wg);
  };
  // The leading tiles every row of the work-group sees in full (complete
  // tiles whose last key is at most its first query), then the rest.
  int T1 = 0;
  if (!ALIBI || (causal && lin_ok)) {
    const int nfull = Lkv / TROWS;
    const int qmin_wg = a.q_pos[q0];
    T1 = causal ? prefix_count(nfull, lane, [&](int u) { return kpos[u * TROWS + TROWS - 1] <= qmin_wg; }) : nfull;
  }
  bool more = true;
  int kv0 = 0, t = 0;
#pragma clang loop unroll(disable)
  for (; more && t < T1; kv0 += TROWS, ++t) more = tile_step(kv0, t, std::true_type{});
#pragma clang loop unroll(disable)
  for (; more; kv0 += TROWS, ++t) more = tile_step(kv0, t, std::false_type{});

  if (!touched) return;
  // dq_acc += scale * dQ; element (dt, e) of this lane is dim 32*dt +
  // 8*(e/4) + 4*hf + e%4 of query `row`. Through a buffer resource from the
  // work-group's first row to the chunk's end (rows past it read zeros and
  // drop their stores), all loads before the first sum.
  const auto rdq = make_rsrc(a.dq + (qhead * Lq + q0) * D, (int64_t)(Lq - q0) * D * 4);
  auto dq_off = [&](int dt, int a4) { return (uint32_t)(((row - q0) * D + 32 * dt + 8 * a4 + 4 * hf) * 4); };
  uint4 old[DT][4];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) old[dt][a4] = buf_load16(rdq, dq_off(dt, a4));
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
      buf_store16(rdq, dq_off(dt, a4), fmaf(a.scale, dQ[dt][4 * a4 + 0], __uint_as_float(old[dt][a4].x)),
                  fmaf(a.scale, dQ[dt][4 * a4 + 1], __uint_as_float(old[dt][a4].y)),
                  fmaf(a.scale, dQ[dt][4 * a4 + 2], __uint_as_float(old[dt][a4].z)),
                  fmaf(a.scale, dQ[dt][4 * a4 + 3], __uint_as_float(old[dt][a4].w)));
  };

  // Persistent walk, as in the forward step: at most two work-groups per CU,
  // split into `groups` groups (work-group i runs on XCD i % 8) that each own
  // a contiguous range of heads, listed head by head with each head's
  // heaviest tiles first (under the causal mask a query tile's work grows
  // with its position) and dealt to the group's work-groups in snake order,
  // so that every work-group gets a similar sum of work and an XCD's
  // work-groups stream the K/V of one head at a time. The arguments reach
  // each tile through a pointer the optimizer cannot see through, so that
  // values derived from them are not held across the walk.
  const int x = (int)blockIdx.x % groups, slot = (int)blockIdx.x / groups;
  const int S = (int)gridDim.x / groups;
  const int hpg = BH / groups;
  const int M = hpg * n_qtiles;
  auto args = [&]() {
    CArgs* ap = (CArgs*)__builtin_amdgcn_kernarg_segment_ptr();  // `a` is the first argument
    asm volatile("" : "+s"(ap));
    return ap;
  };
  for (int k = 0; (k >> 1) * 2 * S < M; ++k) {
    const int i = (k >> 1) * 2 * S + ((k & 1) ? 2 * S - 1 - slot : slot);
    if (i >= M) continue;
    run_task(*args(), (int)threadIdx.x, x * hpg + i / n_qtiles, n_qtiles - 1 - i % n_qtiles);
    __syncthreads();  // the next tile reuses the LDS buffers
  }
}

// CUs of the current device (256 if the runtime cannot say).
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <bool ALIBI>
hipError_t launch_both(const BwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.len_q + 127) / 128;
  const int n_ktiles = (a.len_kv + 127) / 128;
  const int64_t grid_q = (int64_t)n_qtiles * a.batch * a.heads_q;
  const int64_t grid_k = (int64_t)n_ktiles * a.batch * a.heads_kv;
  if (grid_q > INT32_MAX || grid_k > INT32_MAX) return hipErrorInvalidValue;
  // dQ: persistent, two work-groups per CU at most.
  const int bhq = a.batch * a.heads_q;
  const int slots = 2 * cu_count();
  int gq, groups;
  if (grid_q <= slots) {
    gq = (int)grid_q;  // one tile each
    groups = (bhq % 8 == 0) ? 8 : 1;
  } else {
    groups = (bhq % 8 == 0 && slots % 8 == 0) ? 8 : 1;
    gq = slots;
  }
  hipLaunchKernelGGL((bwd_dq_kernel<ALIBI>), dim3((unsigned)gq), dim3(kThreads), 0, stream, a, n_qtiles, groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<ALIBI>), dim3((unsigned)grid_k), dim3(kThreadsKV), 0, stream, a,
                     n_ktiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  return a.slopes ? launch_both<true>(a, stream) : launch_both<false>(a, stream);
}

}  // namespace ra
