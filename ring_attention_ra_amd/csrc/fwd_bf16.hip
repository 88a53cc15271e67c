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
//  * One 512-thread work-group (8 waves) works on 256 query rows of one head
//    at a time; each wave owns 32 rows. K/V stream through LDS in tiles of 64 keys,
//    moved global -> LDS by the DMA path (global_load_lds_dwordx4, no
//    register staging). Rows past the end of the chunk are clamped to the
//    last key and masked.
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
//  * Ping-pong between two sets of four waves (one wave of each set per
//    SIMD): over the tiles that every row of the work-group sees in full,
//    both sets run "MFMA phase | barrier | softmax phase | barrier" with set 1
//    one phase behind set 0, so on each SIMD one wave's matrix products
//    overlap the other wave's exponentials. An MFMA phase is the QK product
//    of the next tile and the P.V product of the current one; its LDS
//    fragment reads run four MFMAs ahead of use, and the wave raises its
//    issue priority for the phase so that its MFMAs and reads are not held
//    behind the other wave's VALU work. Without ALiBi, the fragments of the
//    first four QK products are read at the start of the wave's preceding
//    softmax phase, so the MFMA phase opens with a product instead of an LDS
//    round trip. Under ALiBi (with the causal mask) the QK accumulators of a
//    fully visible tile start from its per-key bias term divided by
//    scale * log2 e, so the softmax adds only a per-row constant.
//    K has four LDS buffers and V three: at the end of its MFMA phase for
//    tile t every wave copies its share of K(t+4) and V(t+2) into the
//    buffers that tiles t and t-1 leave, and waits for its previous step's
//    copies before the barrier, so a copy has two phases to land and a K
//    tile is published a full phase before its first fragments are read
//    early. The copies are issued from inline
//    assembly, invisible to the compiler's wait insertion, so fragment reads
//    of the other buffers go ahead while they fly. Empty volatile asm
//    statements pin each phase's results and scheduling barriers keep the
//    compiler from moving work across the work-group barriers. The
//    remaining tiles (diagonal, ragged, or ALiBi without the causal mask)
//    follow one at a time with all waves in step, double-buffered, with
//    per-element masks where needed.
//  * The output is rescaled lazily: exponents are taken against a reference
//    that is raised to the tile max (and O, l rescaled) only when the scores
//    outgrow it. Over the fully visible tiles without ALiBi no row max is
//    taken at all: the
//    exponentials are computed against the reference first, and only when a
//    lane's sum of P exceeds 2^14 (or the reference is still -inf) does the
//    wave take the max, move the reference and redo them, so P stays below
//    2^14, well inside bf16 / fp32 range. The masked tiles move it when the
//    tile max exceeds it by more than 2^8. The reference is what is stored as
//    m: l = sum exp(s - m) and o_acc = sum exp(s - m) v are taken against it,
//    so m + ln l is the log-sum-exp, and max s - 14 ln 2 <= m <= max s.
//  * Scores are kept in base-2 units (scale * log2 e folded into one FMA) and
//    exponentiated with v_exp_f32; state in memory is in natural units.
//  * Key tiles past the last query of the work-group are never visited
//    (positions increase); a wave skips tiles entirely in its causal future.
//    Under the causal mask the ALiBi term of a fully visible tile is linear
//    in the key position, so it becomes one per-key term staged in LDS (the
//    start value of the QK accumulators in the ping-pong loop) plus one
//    per-row constant.
//  * The launch is persistent: at most one work-group per CU, each walking a
//    fixed list of query tiles, so that no CU waits for a second dispatch.
//    Each XCD's work-groups share a range of whole heads and take them one
//    head at a time (its L2 serves that head's K/V stream to all of them),
//    and each head's tiles are dealt heaviest first in snake order so that
//    every work-group gets a similar sum of work.
//  * K and V tiles are stored as 64-column halves with XOR-swizzled 16-byte
//    chunks, so that neither the K row reads nor the transposing V reads meet
//    a bank conflict and the fragment addresses keep folding into immediate
//    offsets.
#include <type_traits>

#include "tile_common.h"

namespace ra {
namespace {

constexpr int BM = 256;  // query rows per work-group (two sets of 4 waves x 32 rows)
constexpr int BN = kTileRows;  // keys per tile (64)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, base-2 units
constexpr float kLimit = 16384.0f;  // bound on a lane's per-tile sum of P (> 32 * 2^kTau)

enum TileMode { kFast = 0, kAlibiLinear = 1, kExact = 2 };

// Scheduling pattern of one MFMA phase: NQK QK products (one LDS read each)
// followed by NPV P.V products (two transposing LDS reads each). The reads of
// the first four products go first; after product i come the reads of
// product i + 4.
template <int NQK, int NPV, int I>
__device__ __forceinline__ void interleave_qk_step() {
  if constexpr (I < NPV + NQK) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (I + 4 < NPV + NQK) {
      __builtin_amdgcn_sched_group_barrier(0x100, (I + 4 < NQK ? 1 : 2), 0);  // LDS reads
    }
    interleave_qk_step<NQK, NPV, I + 1>();
  }
}
// The same pattern when the fragments of products 0..3 are already in
// registers: the phase opens with its first MFMA.
template <int NQK, int NPV>
__device__ __forceinline__ void interleave_qk_rest() {
  interleave_qk_step<NQK, NPV, 0>();
}
// The pattern when the phase has to read those fragments itself: they go
// first.
template <int NQK, int NPV, int N0 = 4>
__device__ __forceinline__ void interleave_qk_first() {
  // reads of QK products 0..3 (and of the accumulator start values, if any)
  __builtin_amdgcn_sched_group_barrier(0x100, N0, 0);
  interleave_qk_step<NQK, NPV, 0>();
}

// Tile counts of a key chunk with increasing positions kpos:
//   ra = #{u < na : kpos[u*BN] <= ba}         (first key of tile u)
//   rb = #{u < nb : kpos[u*BN + BN - 1] <= bb} (last key of complete tile u)
// Both by a 64-way search run together: each round every lane probes one
// evenly spaced tile of each remaining range, and the ballot of the
// (monotone) answers narrows each range to less than its probe spacing, so
// a range of n tiles takes about log64(n) rounds of one load per lane.
__device__ __forceinline__ void tile_counts(const int* kpos, int na, int ba, int nb, int bb, int lane,
                                            int& ra, int& rb) {
  int alo = 0, ahi = na, blo = 0, bhi = nb;
  while (alo < ahi || blo < bhi) {
    const int as = (ahi - alo + 63) >> 6, bs = (bhi - blo + 63) >> 6;
    const int ap = alo + lane * as, bp = blo + lane * bs;
    const bool aok = ap < ahi, bok = bp < bhi;
    const int ak = aok ? kpos[ap * BN] : 0;
    const int bk = bok ? kpos[bp * BN + BN - 1] : 0;
    const int ac = __builtin_popcountll(__builtin_amdgcn_ballot_w64(aok && ak <= ba));
    const int bc = __builtin_popcountll(__builtin_amdgcn_ballot_w64(bok && bk <= bb));
    if (alo < ahi) {
      const int lo = ac > 0 ? alo + (ac - 1) * as + 1 : alo;
      ahi = min(ahi, alo + ac * as);
      alo = lo;
    }
    if (blo < bhi) {
      const int lo = bc > 0 ? blo + (bc - 1) * bs + 1 : blo;
      bhi = min(bhi, blo + bc * bs);
      blo = lo;
    }
  }
  ra = alo;
  rb = blo;
}

template <int D, bool ALIBI>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(StepArgs a, int n_qtiles, int groups) {
  constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  constexpr int KK = D / 16;            // k-steps of the QK product
  constexpr int DT = D / 32;            // 32-row d tiles of O^T
  constexpr int SLOTS = BN * CPR;       // 16-byte slots in a K (or V) tile
  constexpr int DMA_PER_WAVE = SLOTS / (kWaves * 64);

  __shared__ uint4 Ks[4][SLOTS];
  __shared__ uint4 Vs[3][SLOTS];
  __shared__ __align__(16) int kp[4][BN];
  __shared__ __align__(16) float kb[ALIBI ? 4 : 1][BN];
  // The same per-key term divided by scale * log2 e: the start value of the
  // tile's QK accumulators in the ping-pong loop.
  __shared__ __align__(16) float kbc[ALIBI ? 4 : 1][BN];
  __shared__ int kbase[4];  // position of the first key of the tile in kb[]

  const int BH = a.batch * a.heads_q;

  // One query tile (256 rows of one head) of the step; the work-group walks
  // a list of them (see the loop at the end).
  using CArgs = const __attribute__((address_space(4))) StepArgs;
  auto run_task = [&](CArgs& a, const int tid, const int bh_in, const int qt_in) {
  // Uniform across the work-group; said so, so that addresses derived from them stay scalar.
  const int bh = uniform_i(bh_in), qt = uniform_i(qt_in);
  const int wave = uniform_i(tid >> 6), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int set = wave >> 2;  // two sets of 4 waves, half a tile apart
  const int Lq = a.len_q, Lkv = a.len_kv;
  const int b = bh / a.heads_q, h = bh - b * a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
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

  // Keys past the work-group's last query are never visible (positions
  // increase): when even the first key is, the state stays as it is.
  const int qmax_wg = a.q_pos[min(q0 + BM - 1, Lq - 1)];
  const int qmin_wg = a.q_pos[q0];
  const int n_tiles = (Lkv + BN - 1) / BN;
  if (causal && kpos[0] > qmax_wg) return;

  const int qmin_w = wave_active ? a.q_pos[q0w] : INT32_MAX;
  const int qmax_w = wave_active ? a.q_pos[min(q0w + 31, Lq - 1)] : INT32_MIN;
  const int my_pos = row_ok ? a.q_pos[row] : INT32_MAX;
  const float c = a.scale * RA_LOG2E;
  const bool fast_ok = c > 0.0f;
  const float sl2 = ALIBI ? a.slopes[h] * RA_LOG2E : 0.0f;
  const float sl2c = ALIBI ? a.slopes[h] / a.scale : 0.0f;

  // ---- tile movement ----
  // Phase-1 copies: every wave moves DMA_PER_WAVE 16-byte slots of a K
  // tile and of a V tile (offsets precomputed).
  // K and V tiles share the layout of tile_slot, so one set of source
  // offsets serves both.
  uint32_t d_off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    int r;
    const int ch = tile_slot_chunk((wave * DMA_PER_WAVE + i) * 64 + lane, &r);
    d_off[i] = (uint32_t)(r * D + 8 * ch) * 2;
  }
  auto dma_p1 = [&](int kbuf, int kv0k, int vbuf, int kv0v) {  // complete tiles only
    const char* kt = reinterpret_cast<const char*>(kh + (int64_t)kv0k * D);
    const char* vt = reinterpret_cast<const char*>(vh + (int64_t)kv0v * D);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int base = (wave * DMA_PER_WAVE + i) * 64;
      dma16(kt + d_off[i], &Ks[kbuf][base]);
      dma16(vt + d_off[i], &Vs[vbuf][base]);
    }
    // ALiBi: wave 0 also copies the key positions of the K tile.
    if constexpr (ALIBI) if (wave == 0) dma4(kpos + kv0k + lane, &kp[kbuf][0]);
  };
  // All eight waves; rows past the end of the chunk are clamped to the last
  // key (they are masked).
  auto dma_all = [&](uint4* tile, const uint16_t* src, int kv0) {
    const char* t = reinterpret_cast<const char*>(src + (int64_t)kv0 * D);
    const int last = Lkv - 1 - kv0;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int base = (wave * DMA_PER_WAVE + i) * 64;
      int r;
      const int ch = tile_slot_chunk(base + lane, &r);
      dma16(t + (uint32_t)(min(r, last) * D + 8 * ch) * 2, &tile[base]);
    }
  };
  auto dma_k = [&](int buf, int kv0) { dma_all(Ks[buf], kh, kv0); };
  auto dma_v = [&](int buf, int kv0) { dma_all(Vs[buf], vh, kv0); };
  auto load_kp = [&](int kv0) { return tid < BN ? kpos[min(kv0 + tid, Lkv - 1)] : 0; };
  auto store_kp = [&](int buf, int kv0, int kpv) {
    if (tid < BN) {
      kp[buf][tid] = kpv;
      if constexpr (ALIBI) {
        const int k0 = kpos[kv0];
        kb[buf][tid] = sl2 * (float)(kpv - k0);
        kbc[buf][tid] = sl2c * (float)(kpv - k0);
        if (tid == 0) kbase[buf] = k0;
      }
    }
  };

  // The first tiles of the ping-pong loop are copied right away (clamped to
  // the chunk; a tile past the range found below is copied but never used),
  // then the query and state loads are issued, so that these round trips to
  // memory overlap each other and the tile-range search that follows them.
  // Whatever path runs next waits for the copies before its first barrier.
  const bool p1_possible = fast_ok && (causal || !ALIBI) && Lkv >= BN;
  if (p1_possible) {
    dma_k(0, 0);
    dma_k(1, min(1, n_tiles - 1) * BN);
    dma_k(2, min(2, n_tiles - 1) * BN);
    dma_v(0, 0);
    dma_v(1, min(1, n_tiles - 1) * BN);
  }

  // Incoming m and l of this lane's row (unconditional loads through a
  // buffer resource: rows past the end read 0 and are replaced below).
  const auto rm = make_rsrc(mh, (int64_t)Lq * 4);
  const auto rl = make_rsrc(lh, (int64_t)Lq * 4);
  const float m_in = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (uint32_t)row * 4, 0, 0));
  const float l_in = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)row * 4, 0, 0));

  // Q fragments (B operand of S^T = K Q^T): lane holds query `row`, d slice
  // 16*kk + 8*hf .. +7.
  uint4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = buf_load16(rq, (uint32_t)(row * D + 16 * kk + 8 * hf) * 2);

  // Running state. O^T element (dt, e) of this lane is d = 32*dt + 8*(e/4) +
  // 4*hf + e%4 of query `row`. m_ref: reference of the exponents (base 2).
  // l per half-wave.
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
  float m_ref = row_ok ? m_in * RA_LOG2E : -INFINITY;
  float l_run = (row_ok && hf == 0) ? l_in : 0.0f;
  bool touched = false;

  // Tile range. T: tiles whose first key is at most the work-group's last
  // query (all tiles without the causal mask). T1: leading complete tiles
  // that every row of the work-group sees in full (their last key is at most
  // its first query), taken by the ping-pong loop; T1 <= T.
  int T = n_tiles, T1 = 0;
  if (p1_possible) T1 = Lkv / BN;
  if (causal) tile_counts(kpos, T, qmax_wg, p1_possible ? T1 : 0, qmin_wg, lane, T, T1);

  // V^T fragment for d tile dt and keys kb0 + 8*hf + 0..7 (two transposing
  // reads); K fragment of rows 32*sb + perm_row(lane%32), k-step kk.
  const FragOffsets fo(lane);
  auto v_frag = [&](int buf, int kb0, int dt) { return tile_col_frag(Vs[buf], kb0, dt, fo); };

  // Scores of the tile (two 32-key blocks, S[sb] element e = key 32*sb +
  // 16*(e/8) + 8*hf + e%8) and its bf16 probabilities P[sb][8] for the next
  // MFMA phase.
  ra_f32x16 S[2];
  uint32_t P[2][8];

  // MFMA work of one step: O^T += V^T P^T for the previous tile (from
  // Vs[vb]), then S^T = K Q^T for the current one (from Ks[kbuf]).
  auto pv_mfma = [&](int vb) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 pb = make_uint4(P[sb][4 * ks + 0], P[sb][4 * ks + 1], P[sb][4 * ks + 2], P[sb][4 * ks + 3]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] = ra_mfma32(v_frag(vb, 32 * sb + 16 * ks, dt), pb, O[dt]);
      }
    }
  };
  auto k_frag = [&](int kbuf, int sb, int kk) { return tile_row_frag(Ks[kbuf], 32 * sb, kk, fo); };
  auto qk_mfma = [&](int kbuf) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      ra_f32x16 acc = ra_f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = ra_mfma32(k_frag(kbuf, sb, kk), qf[kk], acc);
      S[sb] = acc;
    }
  };
  // Under ALiBi, over the fully visible tiles: the accumulators start from
  // the tile's per-key term / (scale * log2 e), so that S * c comes out with
  // the key part of the bias already added.
  auto qk_mfma_bias = [&](int kbuf) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const float4* kv = reinterpret_cast<const float4*>(&kbc[kbuf][32 * sb + 8 * hf]);
      const float4 x0 = kv[0], x1 = kv[1], x2 = kv[4], x3 = kv[5];
      ra_f32x16 acc = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                       x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = ra_mfma32(k_frag(kbuf, sb, kk), qf[kk], acc);
      S[sb] = acc;
    }
  };
  // The same product with the fragments of its first kPre MFMAs already in
  // registers (read at the start of the preceding softmax phase).
  constexpr int kPre = 4;
  uint4 kpre[kPre];
  auto qk_mfma_pre = [&](int kbuf) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      ra_f32x16 acc = ra_f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc = ra_mfma32(sb * KK + kk < kPre ? kpre[sb * KK + kk] : k_frag(kbuf, sb, kk), qf[kk], acc);
      S[sb] = acc;
    }
  };

  // Softmax of tile t in place: S -> P (bf16), lazy rescale of O and l.
  // Scores in base 2: S*c for kFast, S (already scaled and biased) otherwise.
  auto exps = [&](auto mode_tag, float off) {
    constexpr int MODE = decltype(mode_tag)::value;
    float psum = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float x0, x1;
        if constexpr (MODE == kFast) {
          x0 = fmaf(S[sb][e], c, off);
          x1 = fmaf(S[sb][e + 1], c, off);
        } else {
          x0 = S[sb][e] + off;
          x1 = S[sb][e + 1] + off;
        }
        const float p0 = __builtin_amdgcn_exp2f(x0);
        const float p1 = __builtin_amdgcn_exp2f(x1);
        psum += p0 + p1;
        P[sb][e >> 1] = ra_pack_bf16(p0, p1);
      }
    }
    return psum;
  };
  // ALiBi terms of a fully visible tile outside the ping-pong loop (linear in
  // the key position): per-key part added here, per-row constant returned.
  auto alibi_linear = [&](int buf) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const float4* kbv = reinterpret_cast<const float4*>(&kb[buf][32 * sb + 8 * hf]);
#pragma unroll
      for (int e8 = 0; e8 < 2; ++e8) {
        const float4 x0 = kbv[4 * e8], x1 = kbv[4 * e8 + 1];
        const float kv8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) S[sb][8 * e8 + i] = fmaf(S[sb][8 * e8 + i], c, kv8[i]);
      }
    }
    // bias = -slope*(pos_q - pos_k) = slope*(pos_k - base) - slope*(pos_q - base)
    return -sl2 * (float)(my_pos - uniform_i(kbase[buf]));
  };
  // Row max of the tile's scores (base 2), over both halves of the wave.
  auto row_max = [&](auto mode_tag, float rowc) {
    constexpr int MODE = decltype(mode_tag)::value;
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, S[sb][e]);
    tmax = fmaxf(tmax, ra_swap_halves(tmax));
    return MODE == kFast ? tmax * c : tmax + rowc;
  };
  // Move the reference to the tile max when that exceeds it by more than
  // 2^tau (always when it is -inf); rescale O; returns the factor for l.
  auto move_ref = [&](float tmax, bool cond) {
    const float nref = tmax > m_ref + kTau ? fmaxf(m_ref, tmax) : m_ref;
    const float alpha = nref == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref - nref);
    if (!cond || __builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
    }
    m_ref = nref;
    return alpha;
  };

  // Fully visible tiles without ALiBi (ping-pong loop): exponents are first
  // taken against the current reference with no row max at all. Only when some lane's sum
  // of P leaves [0, kLimit] (its reference is -inf, or a score rose more
  // than about log2(kLimit / 32) above it) does the wave take the tile max,
  // move the reference and redo the exponents. Since 32 * 2^tau < kLimit, a
  // tile that passes the check never had to move the reference.
  // Under ALiBi the bias rises by about slope * 64 from one tile to the next
  // as the keys approach the queries, so on the steep heads the check would
  // fail on almost every tile and the exponentials would run twice: those
  // tiles take the row max first and move the reference lazily (by 2^tau).
  auto softmax_fast = [&](auto mode_tag, int buf) {
    constexpr int MODE = decltype(mode_tag)::value;
    if constexpr (MODE == kAlibiLinear) {
      // S holds scores / c with the key part of the bias (qk_mfma_bias); the
      // row part is a constant per lane.
      const float rowc = -sl2 * (float)(my_pos - uniform_i(kbase[buf]));
      const float alpha = move_ref(row_max(std::integral_constant<int, kFast>{}, 0.0f) + rowc, true);
      l_run = fmaf(l_run, alpha,
                   exps(std::integral_constant<int, kFast>{}, rowc - (m_ref == -INFINITY ? 0.0f : m_ref)));
    } else {
      float psum = exps(mode_tag, -m_ref);
      if (__builtin_amdgcn_ballot_w64(!(psum <= kLimit))) {
        const float alpha = move_ref(row_max(mode_tag, 0.0f), true);
        psum = exps(mode_tag, m_ref == -INFINITY ? 0.0f : -m_ref);
        l_run *= alpha;
      }
      l_run += psum;
    }
  };

  // Any tile: masked per element where needed, with the row max.
  auto softmax = [&](auto mode_tag, int buf, int kv0) {
    constexpr int MODE = decltype(mode_tag)::value;
    float rowc = 0.0f;
    if constexpr (MODE == kAlibiLinear) {
      rowc = alibi_linear(buf);
    } else if constexpr (MODE == kExact) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int4* kpv = reinterpret_cast<const int4*>(&kp[buf][32 * sb + 8 * hf]);
#pragma unroll
        for (int e8 = 0; e8 < 2; ++e8) {
          const int4 p0 = kpv[4 * e8], p1 = kpv[4 * e8 + 1];
          const int kv8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int j = 32 * sb + 16 * e8 + 8 * hf + i;
            float x = S[sb][8 * e8 + i] * c;
            if (ALIBI) x = fmaf(-sl2, (float)abs(my_pos - kv8[i]), x);
            const bool vis = (kv0 + j < Lkv) && (!causal || kv8[i] <= my_pos);
            S[sb][8 * e8 + i] = vis ? x : -INFINITY;
          }
        }
      }
    }
    const float alpha = move_ref(row_max(mode_tag, rowc), false);
    const float psum = exps(mode_tag, rowc - (m_ref == -INFINITY ? 0.0f : m_ref));
    l_run = fmaf(l_run, alpha, psum);
  };
  constexpr int kUnmasked = ALIBI ? kAlibiLinear : kFast;

  // A work-group barrier that the compiler may not move any instruction
  // across, so that each set's MFMA and softmax phases stay where they are.
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Empty volatile asm that reads and rewrites the values a phase produces:
  // the optimizer may then neither sink that phase's arithmetic past the
  // barrier that follows it nor hoist the next phase's work above it.
  auto pin_softmax = [&]() {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(P[sb][i]));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+v"(O[dt]));
    asm volatile("" : "+v"(l_run), "+v"(m_ref));
  };
  auto pin_mfma = [&]() {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) asm volatile("" : "+v"(S[sb]));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+v"(O[dt]));
  };

  if (T1 > 0) {
    // ---- phase 1: ping-pong. Both sets run the same instruction stream,
    // "MFMA work of step t | barrier | softmax of tile t | barrier", set 1 one
    // phase behind set 0 (one extra barrier at its start, set 0 one at its
    // end), so on every SIMD one set's MFMAs overlap the other set's softmax.
    // Step t's MFMA work is the P.V of tile t-1 and the QK of tile t. Set 0
    // issues the copies at the start of its MFMA phase u: K(u+1) and V(u),
    // waited for at the end of its following softmax phase.
    touched = true;
    // Four K and three V buffers; K tile u lives in K buffer u % 4, V tile u
    // in V buffer u % 3. K(0..2) and V(0..1) were copied up front, K(3) now.
    dma_k(3, min(3, n_tiles - 1) * BN);
    if constexpr (ALIBI) {
#pragma unroll
      for (int u = 0; u < 4; ++u) store_kp(u, min(u, n_tiles - 1) * BN, load_kp(min(u, n_tiles - 1) * BN));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (set == 1) phase_barrier();
    if constexpr (ALIBI) qk_mfma_bias(0); else qk_mfma(0);
    pin_mfma();
    phase_barrier();
    // K buffers of tiles t .. t+3 and V buffers of tiles t-1 .. t+1 (rotating).
    int k0 = 0, k1 = 1, k2 = 2, k3 = 3;
    int v0 = 0, v1 = 1, v2 = 2;
#pragma clang loop unroll(disable)
    for (int t = 0; t < T1; ++t) {
      // First fragments of the next QK product, read before the softmax so
      // that their latency hides behind it. K(t+1) was copied four phases ago
      // and every wave has waited for its share of it before a barrier that
      // both sets have passed since, so the reads may run ahead of the MFMA
      // phase.
      // The ALiBi variant reads its fragments, and its accumulators' start
      // values, in the MFMA phase: the early reads measured 1% slower there.
      if constexpr (!ALIBI) {
#pragma unroll
        for (int i = 0; i < kPre; ++i) kpre[i] = k_frag(k1, i / KK, i % KK);
        __builtin_amdgcn_sched_barrier(0);
      }
      softmax_fast(std::integral_constant<int, kUnmasked>{}, k0);
      pin_softmax();
      phase_barrier();
      __builtin_amdgcn_s_setprio(1);
      // The last QK reads a stale tile and is discarded. LDS fragment reads
      // run four MFMAs ahead of use.
      if constexpr (!ALIBI) {
        qk_mfma_pre(k1);
        pv_mfma(v0);
        interleave_qk_rest<2 * KK, 4 * DT>();
      } else {
        qk_mfma_bias(k1);
        pv_mfma(v0);
        interleave_qk_first<2 * KK, 4 * DT, 12>();
      }
      // Copies: K(t+4) into the buffer K(t) leaves, V(t+2) into the one
      // V(t-1) left (clamped to the last phase-1 tile). Every reader of those
      // buffers has passed a barrier since. This wave's copies of the
      // previous step must land before the barrier; this step's may stay in
      // flight.
      dma_p1(k0, min(t + 4, T1 - 1) * BN, v2, min(t + 2, T1 - 1) * BN);
      pin_mfma();
      __builtin_amdgcn_s_setprio(0);
      // s_waitcnt vmcnt(n), n = this step's copies (expcnt and lgkmcnt fields
      // at their maximum: no wait; vmcnt in bits 3:0).
      if (ALIBI && wave == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DMA_PER_WAVE + 1));
        // Key positions of tile t+3 have landed: its ALiBi terms.
        const int kpv = kp[k3][lane], kf = kp[k3][0];
        kbc[k3][lane] = sl2c * (float)(kpv - kf);
        if (lane == 0) kbase[k3] = kf;
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DMA_PER_WAVE));
      }
      phase_barrier();
      const int kn = k0;
      k0 = k1;
      k1 = k2;
      k2 = k3;
      k3 = kn;
      const int vn = v0;
      v0 = v1;
      v1 = v2;
      v2 = vn;
    }
    if (set == 0) phase_barrier();
  }

  // ---- phase 2: the remaining tiles (diagonal, ragged, or ALiBi without the
  // causal mask), one at a time with all eight waves in step; K, V of tile t
  // in buffer (t - T1) & 1.
  if (T1 < T) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    dma_k(0, T1 * BN);
    dma_v(0, T1 * BN);
    store_kp(0, T1 * BN, load_kp(T1 * BN));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma clang loop unroll(disable)
    for (int t = T1; t < T; ++t) {
      const int buf = (t - T1) & 1, kv0 = t * BN;
      const bool have_next = t + 1 < T;
      int kp_nx = 0;
      if (have_next) {  // that buffer was last read before the previous barrier
        dma_k(buf ^ 1, kv0 + BN);
        dma_v(buf ^ 1, kv0 + BN);
        kp_nx = load_kp(kv0 + BN);
      }
      const int kfirst = uniform_i(kp[buf][0]);
      const int klast = uniform_i(kp[buf][BN - 1]);
      if (wave_active && !(causal && kfirst > qmax_w)) {
        touched = true;
        qk_mfma(buf);
        const bool masked = (kv0 + BN > Lkv) || (causal && klast > qmin_w) || !fast_ok;
        if (masked || (ALIBI && !causal))
          softmax(std::integral_constant<int, kExact>{}, buf, kv0);
        else
          softmax(std::integral_constant<int, kUnmasked>{}, buf, kv0);
        pv_mfma(buf);
      }
      if (!have_next) break;
      store_kp(buf ^ 1, kv0 + BN, kp_nx);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // When the ping-pong loop took every tile its last copies may still be in
  // flight: let them land before the work-group can end and free its LDS.
  __builtin_amdgcn_s_waitcnt(0);
  if (!touched) return;
  // Write the state back, taken against the reference.
  const float l_tot = l_run + ra_swap_halves(l_run);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      buf_store16(ro, (uint32_t)(row * D + 32 * dt + 8 * a4 + 4 * hf) * 4, O[dt][4 * a4 + 0],
                  O[dt][4 * a4 + 1], O[dt][4 * a4 + 2], O[dt][4 * a4 + 3]);
    }
  }
  if (row_ok && hf == 0) {
    mh[row] = m_ref * RA_LN2;
    lh[row] = l_tot;
  }
  };

  // Persistent walk: the grid holds at most one work-group per CU, split into
  // `groups` groups (work-group i runs on XCD i % 8, so with 8 groups each
  // group is one XCD) that each own a contiguous range of heads. A group's
  // query tiles are listed head by head, each head's heaviest first (under
  // the causal mask a tile's work grows with its position), and dealt out to
  // its work-groups in snake order -- forward in even rounds, backward in odd
  // ones. Every work-group then gets a similar sum of work with no second
  // dispatch, and an XCD's work-groups stream the K/V of one head (two at a
  // round boundary) through its L2 together: the step's HBM reads fall from
  // 2.9x to 1.4x its algorithmic reads on the 128K zig-zag share (against 4
  // heads interleaved per XCD).
  const int x = (int)blockIdx.x % groups, slot = (int)blockIdx.x / groups;
  const int S = (int)gridDim.x / groups;
  const int hpg = BH / groups;
  const int M = hpg * n_qtiles;
  // The arguments and the thread index pass through registers that the
  // optimizer cannot see through, once per tile: values derived from them are
  // then computed inside the tile instead of being held in registers across
  // the whole walk.
  auto args = [&]() {
    CArgs* ap = (CArgs*)__builtin_amdgcn_kernarg_segment_ptr();  // `a` is the first argument
    asm volatile("" : "+s"(ap));
    return ap;
  };
  auto thread = [&]() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & (kThreads - 1);
  };
  for (int k = 0; (k >> 1) * 2 * S < M; ++k) {
    const int i = (k >> 1) * 2 * S + ((k & 1) ? 2 * S - 1 - slot : slot);
    if (i >= M) continue;
    run_task(*args(), thread(), x * hpg + i / n_qtiles, n_qtiles - 1 - i % n_qtiles);
    __syncthreads();  // the next tile reuses the LDS buffers
  }
}

// Work-groups of the persistent forward launch: one per CU at most.
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <int D, bool ALIBI>
hipError_t launch_d(const StepArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.len_q + BM - 1) / BM;
  const int64_t tasks = (int64_t)n_qtiles * a.batch * a.heads_q;
  if (tasks > INT32_MAX) return hipErrorInvalidValue;
  const int bh = a.batch * a.heads_q;
  const int ncu = cu_count();
  int grid, groups;
  if (tasks <= ncu) {
    grid = (int)tasks;  // one tile each
    groups = (bh % 8 == 0) ? 8 : 1;
  } else {
    groups = (bh % 8 == 0 && ncu % 8 == 0) ? 8 : 1;
    grid = ncu;
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, ALIBI>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     a, n_qtiles, groups);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const StepArgs& a, hipStream_t stream) {
  const bool alibi = a.slopes != nullptr;
  if (a.head_dim == 128) return alibi ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  return alibi ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
}

}  // namespace ra
