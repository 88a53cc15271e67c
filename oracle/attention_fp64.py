"""Plain fp64 definition of one ring rank's attention share (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module. It imports nothing from the product package.

Notation (B batch, Hq query heads, Hkv key/value heads, S global sequence
length, N ring ranks, C = S / N tokens per rank, D head dimension):

* ``q_g, k_g, v_g`` are global-order arrays ``[B, H, S, D]``; they are the exact
  values the GPU consumes (already rounded to the working dtype), upcast here to
  float64.
* Rank ``r`` holds the query rows at the global positions ``rank_positions``.
* The score of query position p against key position j in query head h is
  ``s_pj = scale * <q_p, k_j> - slope_h * |p - j|`` (ALiBi term only when
  slopes are given), visible iff ``j <= p`` under the causal mask.
* ``O_p = sum_j softmax_j(s_pj) v_j`` and ``LSE_p = ln sum_j exp(s_pj)`` over the
  visible keys, in one pass over every visible key of the row: no chunking and
  no merging. Rows are independent, so rows are grouped into blocks only to
  bound memory; each row's reduction is the plain one.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CONTIGUOUS = "contiguous"
ZIGZAG = "zigzag"


# ---------------------------------------------------------------------------
# Positions and layouts
# ---------------------------------------------------------------------------

def rank_positions(seq_len: int, n_ranks: int, rank: int, layout: str) -> np.ndarray:
    """Global token positions held by ``rank``, in the rank's local row order.

    Contiguous: the sequence is cut along its length into N equal consecutive
    pieces and rank r holds piece r (discosf.com, §2.1 序列切分策略对比, the
    ``torch.split(..., seq_len//4, dim=1)`` split).

    Zig-zag: tokens are dealt out round-robin, GPU 0 holding 0, 4, 8, ... and
    GPU 1 holding 1, 5, 9, ... for four GPUs (digipub.cc, section "Zig Zag Ring
    Attention"), i.e. token i goes to rank i mod N. Local row t is the t-th of
    the rank's tokens in increasing global order (reading: the page fixes the
    set, not the local order; increasing order keeps positions monotone).
    """
    if n_ranks <= 0 or seq_len % n_ranks:
        raise ValueError("seq_len must be a positive multiple of n_ranks")
    if not 0 <= rank < n_ranks:
        raise ValueError("rank out of range")
    c = seq_len // n_ranks
    t = np.arange(c, dtype=np.int64)
    if layout == CONTIGUOUS:
        return rank * c + t
    if layout == ZIGZAG:
        return t * n_ranks + rank
    raise ValueError(f"unknown layout {layout!r}")


def owner_rank(positions: np.ndarray, seq_len: int, n_ranks: int, layout: str) -> np.ndarray:
    """Rank (= ring chunk index) that holds each global position (inverse of
    ``rank_positions``; same passages)."""
    positions = np.asarray(positions, dtype=np.int64)
    if layout == CONTIGUOUS:
        return positions // (seq_len // n_ranks)
    if layout == ZIGZAG:
        return positions % n_ranks
    raise ValueError(f"unknown layout {layout!r}")


def ring_schedule(n_ranks: int, rank: int) -> list[int]:
    """Order in which rank r meets the K/V chunks around the ring.

    Each device first attends with its own K/V, then repeatedly receives the
    chunk of device i-1 and forwards what it holds to i+1 (discosf.com, §3.1
    环形通信拓扑; digipub.cc, section "Zig Zag Ring Attention"). After j hops
    rank r holds the chunk that started on rank (r - j) mod N.
    """
    return [(rank - j) % n_ranks for j in range(n_ranks)]


def permute_to_ranks(x: np.ndarray, n_ranks: int, layout: str) -> np.ndarray:
    """Global order ``[..., S, D]`` -> rank-major ``[N, ..., C, D]`` (row t of
    rank r is global row ``rank_positions(S, N, r, layout)[t]``)."""
    x = np.asarray(x)
    s = x.shape[-2]
    return np.stack([x[..., rank_positions(s, n_ranks, r, layout), :] for r in range(n_ranks)])


def permute_from_ranks(y: np.ndarray, layout: str) -> np.ndarray:
    """Inverse of ``permute_to_ranks``: rank-major ``[N, ..., C, D]`` -> global."""
    y = np.asarray(y)
    n = y.shape[0]
    c = y.shape[-2]
    out = np.empty(y.shape[1:-2] + (n * c, y.shape[-1]), dtype=y.dtype)
    for r in range(n):
        out[..., rank_positions(n * c, n, r, layout), :] = y[r]
    return out


# ---------------------------------------------------------------------------
# ALiBi
# ---------------------------------------------------------------------------

def alibi_slopes(num_heads: int) -> np.ndarray:
    """Per-head ALiBi slopes ``2^(-8 i / H)`` for i = 1..H (intelliparadigm.com,
    §2.1.2 ALiBi方案的创新设计). Head index h (0-based) gets i = h + 1."""
    i = np.arange(1, num_heads + 1, dtype=np.float64)
    return np.exp2(-8.0 * i / num_heads)


# ---------------------------------------------------------------------------
# Forward: accumulator state, finalisation, attention
# ---------------------------------------------------------------------------

def _threads(threads):
    if threads is not None:
        return max(1, int(threads))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _row_block_scores(qb, kh, p, kpos, scale, slope, causal, allowed):
    """Scores of the query rows ``qb`` (positions p) against the keys ``kh``
    (positions kpos), with the ALiBi term and with -inf where a key is not
    visible. ``allowed`` (bool over keys or None) restricts the key set."""
    s = scale * (qb @ kh.T)
    if slope is not None:
        # bias = -slope * |pos_q - pos_k|, added after the 1/sqrt(d) scaling
        # (intelliparadigm.com, §2.1.2: scores + bias with bias = -distance*slopes).
        s = s - slope * np.abs(p[:, None] - kpos[None, :]).astype(np.float64)
    vis = np.ones(s.shape, dtype=bool)
    if causal:
        # A token sees only earlier tokens (digipub.cc, section "Zig Zag Ring
        # Attention"). Reading: its own position counts as visible, otherwise
        # token 0 would see no key at all and its row would be undefined.
        vis &= kpos[None, :] <= p[:, None]
    if allowed is not None:
        vis &= allowed[None, :]
    s[~vis] = -np.inf
    return s


def _prep(q_g, k_g, v_g):
    q_g = np.asarray(q_g)
    k_g = np.asarray(k_g)
    v_g = np.asarray(v_g)
    if q_g.ndim != 4 or k_g.ndim != 4 or v_g.shape != k_g.shape:
        raise ValueError("q_g, k_g, v_g must be [B, H, S, D] with k/v equal")
    b, hq, s, d = q_g.shape
    if k_g.shape[0] != b or k_g.shape[2] != s or k_g.shape[3] != d:
        raise ValueError("q/k shape mismatch")
    hkv = k_g.shape[1]
    if hq % hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return q_g, k_g, v_g, b, hq, hkv, s, d


def accumulator_state(q_g, k_g, v_g, n_ranks, rank, layout, causal, scale,
                      slopes=None, key_chunks=None, rows=None, heads=None,
                      block_rows=256, threads=None):
    """Running state (o_acc, m, l) of rank ``rank`` after it has folded in the
    K/V chunks listed in ``key_chunks`` (all chunks when None).

    The state is the one the pages' online softmax carries (intelliparadigm.com,
    §3.1.2 FlashAttention的核心算法: a running max m, a running sum l and an
    unnormalised output), written here by its definition rather than by any
    update rule: over the visible keys J of a row,
    ``m = max_J s``, ``l = sum_J exp(s - m)``, ``o_acc = sum_J exp(s - m) v``.
    A row with no visible key has m = -inf, l = 0, o_acc = 0.

    Query head h reads key/value head ``h // (Hq / Hkv)`` (grouped-query
    reading; the pages do not describe GQA).

    Returns float64 arrays o_acc ``[B, Hq', R, D]``, m and l ``[B, Hq', R]``,
    where R = len(rows) (local row indices; all C rows by default) and Hq' =
    len(heads) (query heads; all by default).
    """
    q_g, k_g, v_g, b, hq, hkv, s, d = _prep(q_g, k_g, v_g)
    g = hq // hkv
    pos = rank_positions(s, n_ranks, rank, layout)
    rows = np.arange(pos.size) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(hq)) if heads is None else [int(h) for h in heads]
    if slopes is not None:
        slopes = np.asarray(slopes, dtype=np.float64)
        if slopes.shape != (hq,):
            raise ValueError("slopes must have one entry per query head")
    allowed = None
    if key_chunks is not None:
        allowed = np.isin(owner_rank(np.arange(s), s, n_ranks, layout), list(key_chunks))

    o_acc = np.zeros((b, len(heads), rows.size, d), dtype=np.float64)
    m = np.full((b, len(heads), rows.size), -np.inf, dtype=np.float64)
    l = np.zeros((b, len(heads), rows.size), dtype=np.float64)

    def work(task):
        bi, hi, r0 = task
        h = heads[hi]
        rsel = rows[r0:r0 + block_rows]
        p = pos[rsel]
        jmax = int(p.max()) + 1 if causal else s
        kpos = np.arange(jmax, dtype=np.int64)
        kh = np.asarray(k_g[bi, h // g, :jmax], dtype=np.float64)
        vh = np.asarray(v_g[bi, h // g, :jmax], dtype=np.float64)
        qb = np.asarray(q_g[bi, h, p], dtype=np.float64)
        sc = _row_block_scores(qb, kh, p, kpos, scale,
                               None if slopes is None else slopes[h], causal,
                               None if allowed is None else allowed[:jmax])
        mb = sc.max(axis=1)
        shift = np.where(np.isneginf(mb), 0.0, mb)
        e = np.exp(sc - shift[:, None])
        m[bi, hi, r0:r0 + rsel.size] = mb
        l[bi, hi, r0:r0 + rsel.size] = e.sum(axis=1)
        o_acc[bi, hi, r0:r0 + rsel.size] = e @ vh

    tasks = [(bi, hi, r0) for bi in range(b) for hi in range(len(heads))
             for r0 in range(0, rows.size, block_rows)]
    nt = _threads(threads)
    if nt == 1 or len(tasks) == 1:
        for t in tasks:
            work(t)
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            list(ex.map(work, tasks))
    return o_acc, m, l


def finalize_state(o_acc, m, l):
    """O = o_acc / l and LSE = m + ln l (natural log), the normalisation the
    pages apply after the last block (intelliparadigm.com, §3.1.2: output / l).
    A row that saw no key (l = 0) gets O = 0 and LSE = -inf."""
    o_acc = np.asarray(o_acc, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    pos_l = l > 0
    safe = np.where(pos_l, l, 1.0)
    o = np.where(pos_l[..., None], o_acc / safe[..., None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(pos_l, m + np.log(safe), -np.inf)
    return o, lse


def attention_rank_share(q_g, k_g, v_g, n_ranks, rank, layout, causal, scale,
                         slopes=None, key_chunks=None, rows=None, heads=None,
                         block_rows=256, threads=None):
    """Attention output O ``[B, Hq', R, D]`` and LSE ``[B, Hq', R]`` (float64)
    for the local rows of ``rank`` over every visible key (or the keys of the
    chunks in ``key_chunks``). Argument meaning as in ``accumulator_state``."""
    o_acc, m, l = accumulator_state(q_g, k_g, v_g, n_ranks, rank, layout, causal, scale,
                                    slopes, key_chunks, rows, heads, block_rows, threads)
    return finalize_state(o_acc, m, l)


def visible_pairs(seq_len: int, n_ranks: int, rank: int, layout: str, causal: bool) -> int:
    """Number of visible (query, key) pairs per head in the rank's share,
    counted from the positions (each causal row p sees p + 1 keys)."""
    pos = rank_positions(seq_len, n_ranks, rank, layout)
    if not causal:
        return int(pos.size) * seq_len
    return int((pos + 1).sum())


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def attention_rank_share_bwd(q_g, k_g, v_g, do_local, n_ranks, rank, layout, causal, scale,
                             slopes=None, rows=None, keys=None, kv_heads=None,
                             block_rows=64, threads=None):
    """Gradients of ``L = sum_t <O_t, dO_t>`` over the rank's local rows t.

    The pages give no backward formulas beyond recomputing the attention
    matrix from saved statistics instead of storing it (intelliparadigm.com,
    §3.1.2, 重计算策略). This is the textbook softmax-attention gradient, with
    ``P_pj = exp(s_pj - LSE_p)`` recomputed from the oracle's own LSE:

    * ``Delta_p = <dO_p, O_p>``
    * ``dV_j = sum_p P_pj dO_p``
    * ``dS_pj = P_pj (<dO_p, v_j> - Delta_p)``
    * ``dQ_p = scale * sum_j dS_pj k_j``
    * ``dK_j = scale * sum_p dS_pj q_p``

    The ALiBi term is a constant and has no gradient. Key/value gradients sum
    the query heads that share a key/value head.

    ``do_local`` is ``[B, Hq, C, D]`` in local row order. Returns
    ``dq [B, Hq', R, D]`` for local rows ``rows`` (all by default) and query
    heads in the groups of ``kv_heads``, and ``dk, dv [B, Hkv', K, D]`` for the
    global key positions ``keys`` (all S by default), all float64.
    """
    q_g, k_g, v_g, b, hq, hkv, s, d = _prep(q_g, k_g, v_g)
    g = hq // hkv
    do_local = np.asarray(do_local)
    c = s // n_ranks
    if do_local.shape != (b, hq, c, d):
        raise ValueError("do_local must be [B, Hq, C, D]")
    pos = rank_positions(s, n_ranks, rank, layout)
    rows = np.arange(c) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(s) if keys is None else np.asarray(keys, dtype=np.int64)
    kv_heads = list(range(hkv)) if kv_heads is None else [int(h) for h in kv_heads]
    qheads = [hk * g + i for hk in kv_heads for i in range(g)]
    if slopes is not None:
        slopes = np.asarray(slopes, dtype=np.float64)

    dq = np.zeros((b, len(qheads), rows.size, d), dtype=np.float64)
    dk = np.zeros((b, len(kv_heads), keys.size, d), dtype=np.float64)
    dv = np.zeros((b, len(kv_heads), keys.size, d), dtype=np.float64)
    want_keys = keys.size > 0

    def head_work(task):
        bi, qi = task
        h = qheads[qi]
        hk = h // g
        slope = None if slopes is None else slopes[h]
        kh_all = np.asarray(k_g[bi, hk], dtype=np.float64)
        vh_all = np.asarray(v_g[bi, hk], dtype=np.float64)
        # Rows whose gradients we need: the requested dQ rows, and every local
        # row that can see a requested key (dK_j sums over the rows p that see
        # key j; under the causal mask a row p < min(keys) adds exact zeros).
        if want_keys:
            sees = pos >= keys.min() if causal else np.ones(c, dtype=bool)
            need_rows = np.union1d(np.nonzero(sees)[0], rows)
        else:
            need_rows = rows
        dk_part = np.zeros((keys.size, d))
        dv_part = np.zeros((keys.size, d))
        dq_rows = {}
        for r0 in range(0, need_rows.size, block_rows):
            rsel = need_rows[r0:r0 + block_rows]
            p = pos[rsel]
            jmax = int(p.max()) + 1 if causal else s
            kpos = np.arange(jmax, dtype=np.int64)
            kh = kh_all[:jmax]
            vh = vh_all[:jmax]
            qb = np.asarray(q_g[bi, h, p], dtype=np.float64)
            dob = np.asarray(do_local[bi, h, rsel], dtype=np.float64)
            sc = _row_block_scores(qb, kh, p, kpos, scale, slope, causal, None)
            mb = sc.max(axis=1)
            shift = np.where(np.isneginf(mb), 0.0, mb)
            e = np.exp(sc - shift[:, None])
            lsum = e.sum(axis=1)
            lse = np.where(lsum > 0, shift + np.log(np.where(lsum > 0, lsum, 1.0)), -np.inf)
            pm = np.exp(sc - np.where(np.isneginf(lse), 0.0, lse)[:, None])
            o = pm @ vh
            delta = (dob * o).sum(axis=1)
            dp = dob @ vh.T
            ds = pm * (dp - delta[:, None])
            dq_rows_blk = scale * (ds @ kh)
            for i, t in enumerate(rsel):
                dq_rows[int(t)] = dq_rows_blk[i]
            if want_keys:
                sel = keys < jmax
                kk = keys[sel]
                dk_part[sel] += scale * (ds[:, kk].T @ qb)
                dv_part[sel] += pm[:, kk].T @ dob
        for i, t in enumerate(rows):
            dq[bi, qi, i] = dq_rows[int(t)]
        return bi, kv_heads.index(hk), dk_part, dv_part

    tasks = [(bi, qi) for bi in range(b) for qi in range(len(qheads))]
    nt = _threads(threads)
    if nt == 1 or len(tasks) == 1:
        results = [head_work(t) for t in tasks]
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            results = list(ex.map(head_work, tasks))
    for bi, hki, dkp, dvp in results:
        dk[bi, hki] += dkp
        dv[bi, hki] += dvp
    return dq, dk, dv


__all__ = [
    "CONTIGUOUS", "ZIGZAG", "rank_positions", "owner_rank", "ring_schedule",
    "permute_to_ranks", "permute_from_ranks", "alibi_slopes", "accumulator_state",
    "finalize_state", "attention_rank_share", "attention_rank_share_bwd", "visible_pairs",
]
