"""Pins for the fp64 oracle: checks against facts fixed outside the oracle.

* the pages' worked zig-zag example and the contiguous torch.split (golden),
* the ALiBi slope formula at exact powers of two (golden),
* brute force in pure Python with math.fsum on tiny inputs, with positions
  derived from "token i goes to rank i mod N" rather than the oracle's formula,
* torch's fp64 scaled_dot_product_attention (an independent softmax
  attention) and its autograd for the backward,
* closed forms (zero keys, constant values, the first causal row, the ALiBi
  geometric series),
* invariants (chunked log-sum-exp merge equals one pass, with the pages' two
  flawed merges as negative controls; zig-zag equals contiguous after
  un-permuting; causality; slope 0 equals no bias),
* central finite differences for the backward,
* planted mistakes in the oracle that at least one pin must catch.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_fp64 as ofp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# positions, layouts, permutation
# ---------------------------------------------------------------------------

def test_zigzag_worked_example():
    rows = _golden_rows("zigzag_positions_n4.txt")
    assert rows
    for n, r, *first in rows:
        n, r = int(n), int(r)
        pos = oracle.rank_positions(16 * n, n, r, oracle.ZIGZAG)
        assert pos[: len(first)].tolist() == [int(x) for x in first]


@pytest.mark.parametrize("s,n", [(16, 4), (256, 4), (96, 8), (7, 7)])
def test_contiguous_is_torch_split(s, n):
    chunks = torch.split(torch.arange(s), s // n, dim=0)
    for r in range(n):
        assert oracle.rank_positions(s, n, r, oracle.CONTIGUOUS).tolist() == chunks[r].tolist()


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
@pytest.mark.parametrize("s,n", [(16, 4), (64, 8), (48, 3)])
def test_positions_partition_and_owner(layout, s, n):
    seen = np.zeros(s, dtype=int)
    for r in range(n):
        pos = oracle.rank_positions(s, n, r, layout)
        assert np.all(np.diff(pos) > 0)  # strictly increasing local order
        seen[pos] += 1
        assert np.all(oracle.owner_rank(pos, s, n, layout) == r)
        if layout == oracle.ZIGZAG:
            assert np.all(pos % n == r)  # token i -> rank i mod N
    assert np.all(seen == 1)


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
def test_permute_roundtrip_bitwise(layout):
    x = _rand((2, 3, 24, 5), 1).astype(np.float32)
    y = oracle.permute_to_ranks(x, 4, layout)
    assert y.shape == (4, 2, 3, 6, 5)
    back = oracle.permute_from_ranks(y, layout)
    assert back.tobytes() == x.tobytes()
    for r in range(4):
        pos = oracle.rank_positions(24, 4, r, layout)
        assert np.array_equal(y[r], x[:, :, pos, :])


def test_ring_schedule_visits_each_chunk_once():
    for n in (1, 2, 4, 8, 64):
        for r in range(n):
            sched = oracle.ring_schedule(n, r)
            assert sched[0] == r
            assert sorted(sched) == list(range(n))
            # each hop receives the chunk of the previous device
            for j in range(1, n):
                assert sched[j] == (sched[j - 1] - 1) % n


def test_alibi_slopes_golden():
    for h_total, i, val in _golden_rows("alibi_slopes.txt"):
        sl = oracle.alibi_slopes(int(h_total))
        assert sl[int(i) - 1] == float(val)
    sl = oracle.alibi_slopes(64)
    assert np.all(np.diff(sl) < 0) and sl.shape == (64,)


def test_visible_pairs_counts():
    # closed forms: contiguous r*C^2 + C(C+1)/2 ; zig-zag N*C(C-1)/2 + C(r+1)
    for (s, n) in [(256, 4), (16384, 8), (131072, 8), (65536, 4)]:
        c = s // n
        for r in (0, n - 1):
            assert oracle.visible_pairs(s, n, r, oracle.CONTIGUOUS, True) == r * c * c + c * (c + 1) // 2
            assert oracle.visible_pairs(s, n, r, oracle.ZIGZAG, True) == n * c * (c - 1) // 2 + c * (r + 1)
    assert oracle.visible_pairs(256, 4, 2, oracle.CONTIGUOUS, True) == 10272


# ---------------------------------------------------------------------------
# brute force (pure Python, math.fsum) on tiny inputs
# ---------------------------------------------------------------------------

def _brute(qg, kg, vg, n, r, layout, causal, scale, slopes):
    b_, hq, s, d = qg.shape
    g = hq // kg.shape[1]
    c = s // n
    if layout == oracle.CONTIGUOUS:
        rows = list(range(r * c, (r + 1) * c))
    else:
        rows = [i for i in range(s) if i % n == r]
    o = np.zeros((b_, hq, c, d))
    lse = np.zeros((b_, hq, c))
    for b in range(b_):
        for h in range(hq):
            for t, p in enumerate(rows):
                sc = []
                for j in range(s):
                    if causal and j > p:
                        continue
                    v = scale * math.fsum(float(qg[b, h, p, i]) * float(kg[b, h // g, j, i]) for i in range(d))
                    if slopes is not None:
                        v -= float(slopes[h]) * abs(p - j)
                    sc.append((j, v))
                mx = max(v for _, v in sc)
                w = [(j, math.exp(v - mx)) for j, v in sc]
                z = math.fsum(x for _, x in w)
                for i in range(d):
                    o[b, h, t, i] = math.fsum(x * float(vg[b, h // g, j, i]) for j, x in w) / z
                lse[b, h, t] = mx + math.log(z)
    return o, lse


@pytest.mark.parametrize("layout,causal,alibi,hq,hkv,n", [
    (oracle.CONTIGUOUS, True, False, 2, 2, 2),
    (oracle.ZIGZAG, True, False, 2, 2, 4),
    (oracle.ZIGZAG, False, False, 2, 1, 2),
    (oracle.CONTIGUOUS, True, True, 4, 2, 4),
    (oracle.ZIGZAG, True, True, 4, 1, 2),
    (oracle.CONTIGUOUS, False, True, 2, 2, 2),
])
def test_bruteforce_tiny(layout, causal, alibi, hq, hkv, n):
    s, d = 8, 3
    qg = _rand((1, hq, s, d), 10)
    kg = _rand((1, hkv, s, d), 11)
    vg = _rand((1, hkv, s, d), 12)
    slopes = oracle.alibi_slopes(hq) if alibi else None
    scale = 1 / math.sqrt(d)
    for r in range(n):
        o, lse = oracle.attention_rank_share(qg, kg, vg, n, r, layout, causal, scale, slopes)
        ob, lb = _brute(qg, kg, vg, n, r, layout, causal, scale, slopes)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# torch fp64 SDPA (an independent softmax attention)
# ---------------------------------------------------------------------------

def _sdpa_global(qg, kg, vg, causal, scale, slopes):
    q = torch.from_numpy(qg)
    g = qg.shape[1] // kg.shape[1]
    k = torch.from_numpy(kg).repeat_interleave(g, dim=1)
    v = torch.from_numpy(vg).repeat_interleave(g, dim=1)
    s = qg.shape[2]
    if slopes is None:
        return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale).numpy()
    idx = torch.arange(s, dtype=torch.float64)
    dist = (idx[:, None] - idx[None, :]).abs()
    mask = -torch.from_numpy(np.asarray(slopes))[:, None, None] * dist
    if causal:
        mask = mask.masked_fill(torch.triu(torch.ones(s, s, dtype=torch.bool), 1), float("-inf"))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None], scale=scale).numpy()


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
@pytest.mark.parametrize("causal,alibi,hq,hkv", [(True, False, 4, 4), (True, True, 8, 2),
                                                  (False, False, 4, 1), (False, True, 2, 2)])
def test_matches_torch_sdpa_fp64(layout, causal, alibi, hq, hkv):
    s, n, d = 64, 4, 16
    qg = _rand((2, hq, s, d), 20)
    kg = _rand((2, hkv, s, d), 21)
    vg = _rand((2, hkv, s, d), 22)
    slopes = oracle.alibi_slopes(hq) if alibi else None
    ref = _sdpa_global(qg, kg, vg, causal, 0.25, slopes)
    for r in range(n):
        o, _ = oracle.attention_rank_share(qg, kg, vg, n, r, layout, causal, 0.25, slopes, block_rows=5)
        pos = oracle.rank_positions(s, n, r, layout)
        np.testing.assert_allclose(o, ref[:, :, pos], rtol=0, atol=1e-12)


def test_row_and_head_subsets_match_full():
    s, n, d = 64, 4, 8
    qg, kg, vg = _rand((1, 4, s, d), 1), _rand((1, 2, s, d), 2), _rand((1, 2, s, d), 3)
    o, lse = oracle.attention_rank_share(qg, kg, vg, n, 3, oracle.ZIGZAG, True, 0.3, oracle.alibi_slopes(4))
    rows, heads = [0, 5, 15], [3, 1]
    o2, l2 = oracle.attention_rank_share(qg, kg, vg, n, 3, oracle.ZIGZAG, True, 0.3, oracle.alibi_slopes(4),
                                         rows=rows, heads=heads)
    np.testing.assert_array_equal(o2, o[:, heads][:, :, rows])
    np.testing.assert_array_equal(l2, lse[:, heads][:, :, rows])


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
@pytest.mark.parametrize("causal", [True, False])
def test_zero_keys_give_mean_of_values(layout, causal):
    s, n, d = 32, 4, 6
    qg = _rand((1, 2, s, d), 30)
    kg = np.zeros((1, 2, s, d))
    vg = _rand((1, 2, s, d), 31)
    for r in range(n):
        o, lse = oracle.attention_rank_share(qg, kg, vg, n, r, layout, causal, 0.5)
        pos = oracle.rank_positions(s, n, r, layout)
        for t, p in enumerate(pos):
            cnt = p + 1 if causal else s
            np.testing.assert_allclose(o[0, :, t], vg[0, :, :cnt].mean(axis=1), rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[0, :, t], math.log(cnt), rtol=0, atol=1e-14)


def test_constant_values_and_first_row():
    s, n, d = 32, 4, 6
    qg, kg = _rand((1, 1, s, d), 40), _rand((1, 1, s, d), 41)
    vg = np.full((1, 1, s, d), 1.75)
    o, _ = oracle.attention_rank_share(qg, kg, vg, n, 2, oracle.ZIGZAG, True, 0.4)
    np.testing.assert_allclose(o, 1.75, rtol=0, atol=1e-14)
    vg = _rand((1, 1, s, d), 42)
    o, lse = oracle.attention_rank_share(qg, kg, vg, n, 0, oracle.CONTIGUOUS, True, 0.4)
    # the first causal row sees only itself
    np.testing.assert_allclose(o[0, 0, 0], vg[0, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.4 * float(qg[0, 0, 0] @ kg[0, 0, 0]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
def test_alibi_geometric_series(layout):
    # Q = 0 makes every dot product vanish, so the causal weights of row p are
    # exp(-slope (p - j)) for j <= p: a geometric series with a closed-form sum.
    s, n, h = 16, 4, 4
    qg = np.zeros((1, h, s, s))
    kg = _rand((1, h, s, s), 50)
    vg = np.broadcast_to(np.eye(s), (1, h, s, s)).copy()  # value j is the one-hot e_j
    sl = oracle.alibi_slopes(h)
    for r in range(n):
        o, lse = oracle.attention_rank_share(qg, kg, vg, n, r, layout, True, 1.0, sl)
        for t, p in enumerate(oracle.rank_positions(s, n, r, layout)):
            for hh in range(h):
                a = sl[hh]
                z = math.expm1(-a * (p + 1)) / math.expm1(-a)
                assert abs(lse[0, hh, t] - math.log(z)) < 1e-14
                w = np.array([math.exp(-a * (p - j)) / z if j <= p else 0.0 for j in range(s)])
                np.testing.assert_allclose(o[0, hh, t], w, rtol=0, atol=1e-14)


def test_alibi_symmetric_without_mask():
    s, h = 12, 2
    qg = np.zeros((1, h, s, s))
    vg = np.broadcast_to(np.eye(s), (1, h, s, s)).copy()
    sl = oracle.alibi_slopes(h)
    o, _ = oracle.attention_rank_share(qg, _rand((1, h, s, s), 5), vg, 3, 1, oracle.CONTIGUOUS, False, 1.0, sl)
    for t, p in enumerate(oracle.rank_positions(s, 3, 1, oracle.CONTIGUOUS)):
        for hh in range(h):
            w = np.exp(-sl[hh] * np.abs(p - np.arange(s)))
            np.testing.assert_allclose(o[0, hh, t], w / w.sum(), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def _merge_textbook(states):
    o, m, l = states[0]
    for ob, mb, lb in states[1:]:
        mn = np.maximum(m, mb)
        sh = np.where(np.isneginf(mn), 0.0, mn)
        a, bb = np.exp(m - sh), np.exp(mb - sh)
        o = o * a[..., None] + ob * bb[..., None]
        l = l * a + lb * bb
        m = mn
    return o, m, l


def _merge_page_update(states):
    # The page's online-softmax update rescales the old state by exp(m - new_m)
    # but adds the new block's unnormalised sums without exp(m_blk - new_m).
    o, m, l = states[0]
    for ob, mb, lb in states[1:]:
        mn = np.maximum(m, mb)
        sh = np.where(np.isneginf(mn), 0.0, mn)
        a = np.exp(m - sh)
        o = o * a[..., None] + ob
        l = l * a + lb
        m = mn
    return o, m, l


def _sum_of_normalised(states):
    # Normalise each block separately and add the results (the paged and
    # memory-optimised snippets on the same page do this).
    out = 0
    for ob, mb, lb in states:
        out = out + np.where(lb[..., None] > 0, ob / np.where(lb > 0, lb, 1)[..., None], 0.0)
    return out


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
@pytest.mark.parametrize("alibi", [False, True])
def test_chunked_lse_merge_equals_single_pass(layout, alibi):
    s, n, d, hq = 64, 4, 8, 4
    qg, kg, vg = _rand((1, hq, s, d), 60), _rand((1, 2, s, d), 61), _rand((1, 2, s, d), 62)
    sl = oracle.alibi_slopes(hq) if alibi else None
    for r in range(n):
        o_ref, lse_ref = oracle.attention_rank_share(qg, kg, vg, n, r, layout, True, 0.35, sl)
        states = [oracle.accumulator_state(qg, kg, vg, n, r, layout, True, 0.35, sl, key_chunks=[c])
                  for c in oracle.ring_schedule(n, r)]
        o, lse = oracle.finalize_state(*_merge_textbook(states))
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
        # partial rings: merged state after the first j chunks == restricted attention
        for j in range(1, n):
            o_j, l_j = oracle.finalize_state(*_merge_textbook(states[:j]))
            o_r, l_r = oracle.attention_rank_share(qg, kg, vg, n, r, layout, True, 0.35, sl,
                                                   key_chunks=oracle.ring_schedule(n, r)[:j])
            np.testing.assert_allclose(o_j, o_r, rtol=0, atol=1e-12)
            np.testing.assert_array_equal(np.isneginf(l_j), np.isneginf(l_r))
        # negative controls: the two flawed merges from the pages must disagree
        if r == n - 1:
            o_bad, _ = oracle.finalize_state(*_merge_page_update(states))
            assert np.max(np.abs(o_bad - o_ref)) > 1e-2
            assert np.max(np.abs(_sum_of_normalised(states) - o_ref)) > 1e-2


@pytest.mark.parametrize("alibi", [False, True])
def test_zigzag_equals_contiguous_equals_global(alibi):
    s, n, d, hq = 48, 4, 8, 2
    qg, kg, vg = _rand((1, hq, s, d), 70), _rand((1, hq, s, d), 71), _rand((1, hq, s, d), 72)
    sl = oracle.alibi_slopes(hq) if alibi else None
    glob = {}
    for layout in (oracle.CONTIGUOUS, oracle.ZIGZAG):
        per = [oracle.attention_rank_share(qg, kg, vg, n, r, layout, True, 0.3, sl) for r in range(n)]
        o = oracle.permute_from_ranks(np.stack([p[0] for p in per]), layout)
        lse = oracle.permute_from_ranks(np.stack([p[1][..., None] for p in per]), layout)[..., 0]
        glob[layout] = (o, lse)
    np.testing.assert_allclose(glob[oracle.ZIGZAG][0], glob[oracle.CONTIGUOUS][0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(glob[oracle.ZIGZAG][1], glob[oracle.CONTIGUOUS][1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(glob[oracle.ZIGZAG][0], _sdpa_global(qg, kg, vg, True, 0.3, sl), rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
def test_causal_row_never_sees_later_positions(layout):
    s, n, d = 64, 4, 8
    qg, kg, vg = _rand((1, 2, s, d), 80), _rand((1, 2, s, d), 81), _rand((1, 2, s, d), 82)
    r = 1
    pos = oracle.rank_positions(s, n, r, layout)
    o, lse = oracle.attention_rank_share(qg, kg, vg, n, r, layout, True, 0.3, oracle.alibi_slopes(2))
    cut = int(pos[7])
    kg2, vg2 = kg.copy(), vg.copy()
    kg2[:, :, cut + 1:] = _rand(kg2[:, :, cut + 1:].shape, 83) * 100
    vg2[:, :, cut + 1:] = 1e6
    o2, l2 = oracle.attention_rank_share(qg, kg2, vg2, n, r, layout, True, 0.3, oracle.alibi_slopes(2))
    keep = pos <= cut
    assert o[:, :, keep].tobytes() == o2[:, :, keep].tobytes()
    assert lse[:, :, keep].tobytes() == l2[:, :, keep].tobytes()
    assert not np.allclose(o[:, :, ~keep], o2[:, :, ~keep])


def test_alibi_slope_zero_is_plain_attention_bitwise():
    s, n, d = 32, 4, 8
    qg, kg, vg = _rand((1, 3, s, d), 90), _rand((1, 3, s, d), 91), _rand((1, 3, s, d), 92)
    for layout, causal in itertools.product((oracle.CONTIGUOUS, oracle.ZIGZAG), (True, False)):
        a = oracle.attention_rank_share(qg, kg, vg, n, 2, layout, causal, 0.3, None)
        b = oracle.attention_rank_share(qg, kg, vg, n, 2, layout, causal, 0.3, np.zeros(3))
        assert a[0].tobytes() == b[0].tobytes() and a[1].tobytes() == b[1].tobytes()


def test_empty_rows_in_a_partial_ring():
    # contiguous rank 0 against chunk 1 under the causal mask: no key is visible
    s, n, d = 32, 4, 4
    qg, kg, vg = _rand((1, 1, s, d), 1), _rand((1, 1, s, d), 2), _rand((1, 1, s, d), 3)
    o_acc, m, l = oracle.accumulator_state(qg, kg, vg, n, 0, oracle.CONTIGUOUS, True, 0.5, key_chunks=[1])
    assert np.all(np.isneginf(m)) and np.all(l == 0) and np.all(o_acc == 0)
    o, lse = oracle.finalize_state(o_acc, m, l)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # zig-zag rank 1 against chunk 2: local row 0 (position 1) sees nothing, row 1 sees key 2
    o_acc, m, l = oracle.accumulator_state(qg, kg, vg, n, 1, oracle.ZIGZAG, True, 0.5, key_chunks=[2])
    assert np.isneginf(m[0, 0, 0]) and l[0, 0, 0] == 0
    assert np.all(l[0, 0, 1:] > 0)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _loss(qg, kg, vg, do, n, r, layout, causal, scale, sl):
    o, _ = oracle.attention_rank_share(qg, kg, vg, n, r, layout, causal, scale, sl, threads=1)
    return float((o * do).sum())


@pytest.mark.parametrize("layout,causal,alibi", [(oracle.ZIGZAG, True, False), (oracle.CONTIGUOUS, True, True),
                                                 (oracle.ZIGZAG, False, True)])
def test_bwd_finite_differences(layout, causal, alibi):
    s, n, d, hq, hkv = 8, 2, 3, 2, 1
    qg, kg, vg = _rand((1, hq, s, d), 100), _rand((1, hkv, s, d), 101), _rand((1, hkv, s, d), 102)
    r = 1
    do = _rand((1, hq, s // n, d), 103)
    sl = oracle.alibi_slopes(hq) if alibi else None
    dq, dk, dv = oracle.attention_rank_share_bwd(qg, kg, vg, do, n, r, layout, causal, 0.6, sl)
    pos = oracle.rank_positions(s, n, r, layout)
    eps = 1e-6
    rng = np.random.default_rng(7)
    for _ in range(12):
        which = rng.integers(3)
        arr = (qg, kg, vg)[which]
        idx = tuple(int(rng.integers(x)) for x in arr.shape)
        if which == 0:
            idx = (idx[0], idx[1], int(pos[idx[2] % pos.size]), idx[3])
        plus, minus = arr.copy(), arr.copy()
        plus[idx] += eps
        minus[idx] -= eps
        args = [qg, kg, vg]
        args[which] = plus
        lp = _loss(*args, do, n, r, layout, causal, 0.6, sl)
        args[which] = minus
        lm = _loss(*args, do, n, r, layout, causal, 0.6, sl)
        fd = (lp - lm) / (2 * eps)
        if which == 0:
            t = int(np.nonzero(pos == idx[2])[0][0])
            an = dq[idx[0], idx[1], t, idx[3]]
        else:
            an = (dk, dv)[which - 1][idx]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, idx, fd, an)


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.ZIGZAG])
@pytest.mark.parametrize("alibi,hq,hkv", [(False, 4, 4), (True, 4, 2)])
def test_bwd_matches_torch_autograd(layout, alibi, hq, hkv):
    s, n, d = 32, 4, 8
    qg, kg, vg = _rand((1, hq, s, d), 110), _rand((1, hkv, s, d), 111), _rand((1, hkv, s, d), 112)
    sl = oracle.alibi_slopes(hq) if alibi else None
    r = 2
    pos = oracle.rank_positions(s, n, r, layout)
    do = _rand((1, hq, s // n, d), 113)
    q = torch.from_numpy(qg).requires_grad_()
    k = torch.from_numpy(kg).requires_grad_()
    v = torch.from_numpy(vg).requires_grad_()
    g = hq // hkv
    idx = torch.arange(s, dtype=torch.float64)
    mask = torch.zeros(hq, s, s, dtype=torch.float64)
    if sl is not None:
        mask = -torch.from_numpy(sl)[:, None, None] * (idx[:, None] - idx[None, :]).abs()
    mask = mask.masked_fill(torch.triu(torch.ones(s, s, dtype=torch.bool), 1), float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(g, 1), v.repeat_interleave(g, 1), attn_mask=mask[None], scale=0.45)
    (out[:, :, torch.from_numpy(pos)] * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = oracle.attention_rank_share_bwd(qg, kg, vg, do, n, r, layout, True, 0.45, sl, block_rows=3)
    np.testing.assert_allclose(dq, q.grad.numpy()[:, :, pos], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, k.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, v.grad.numpy(), rtol=0, atol=1e-12)


def test_bwd_subsets_match_full():
    s, n, d = 32, 4, 4
    qg, kg, vg = _rand((1, 4, s, d), 120), _rand((1, 2, s, d), 121), _rand((1, 2, s, d), 122)
    do = _rand((1, 4, s // n, d), 123)
    full = oracle.attention_rank_share_bwd(qg, kg, vg, do, n, 3, oracle.ZIGZAG, True, 0.5)
    rows, keys = np.array([0, 3, 7]), np.array([1, 9, 30, 31])
    sub = oracle.attention_rank_share_bwd(qg, kg, vg, do, n, 3, oracle.ZIGZAG, True, 0.5,
                                          rows=rows, keys=keys, kv_heads=[1])
    np.testing.assert_allclose(sub[0], full[0][:, 2:4][:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sub[1], full[1][:, 1:2][:, :, keys], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sub[2], full[2][:, 1:2][:, :, keys], rtol=0, atol=1e-14)
    # late keys only: rows that cannot see them are skipped, the result is unchanged
    late = np.array([27, 30, 31])
    sub = oracle.attention_rank_share_bwd(qg, kg, vg, do, n, 3, oracle.ZIGZAG, True, 0.5, rows=rows, keys=late)
    np.testing.assert_allclose(sub[1], full[1][:, :, late], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sub[2], full[2][:, :, late], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above
# ---------------------------------------------------------------------------

def _pins_hold():
    checks = [
        test_zigzag_worked_example,
        test_alibi_slopes_golden,
        lambda: test_bruteforce_tiny(oracle.ZIGZAG, True, True, 4, 2, 2),
        lambda: test_bruteforce_tiny(oracle.CONTIGUOUS, True, True, 4, 2, 4),
        lambda: test_matches_torch_sdpa_fp64(oracle.ZIGZAG, True, True, 8, 2),
        lambda: test_constant_values_and_first_row(),
        lambda: test_alibi_geometric_series(oracle.ZIGZAG),
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def _scores_strict_causal(qb, kh, p, kpos, scale, slope, causal, allowed):
    s = scale * (qb @ kh.T)
    if slope is not None:
        s = s - slope * np.abs(p[:, None] - kpos[None, :])
    vis = kpos[None, :] < p[:, None] if causal else np.ones(s.shape, bool)
    s = np.where(vis, s, -np.inf)
    return s


def _scores_signed_alibi(qb, kh, p, kpos, scale, slope, causal, allowed):
    s = scale * (qb @ kh.T)
    if slope is not None:
        s = s + slope * (p[:, None] - kpos[None, :])
    if causal:
        s = np.where(kpos[None, :] <= p[:, None], s, -np.inf)
    return s


def _scores_unscaled_bias(qb, kh, p, kpos, scale, slope, causal, allowed):
    s = qb @ kh.T
    if slope is not None:
        s = s - slope * np.abs(p[:, None] - kpos[None, :])
    s = scale * s
    if causal:
        s = np.where(kpos[None, :] <= p[:, None], s, -np.inf)
    return s


def _positions_reversed(seq_len, n_ranks, rank, layout):
    c = seq_len // n_ranks
    t = np.arange(c)
    return rank * c + t if layout == oracle.CONTIGUOUS else (c - 1 - t) * n_ranks + rank


def _alibi_zero_based(num_heads):
    return np.exp2(-8.0 * np.arange(num_heads) / num_heads)


def test_pins_hold_for_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("name,replacement", [
    ("_row_block_scores", _scores_strict_causal),
    ("_row_block_scores", _scores_signed_alibi),
    ("_row_block_scores", _scores_unscaled_bias),
    ("rank_positions", _positions_reversed),
    ("alibi_slopes", _alibi_zero_based),
])
def test_planted_mistake_is_caught(monkeypatch, name, replacement):
    monkeypatch.setattr(ofp, name, replacement)
    if name in ("rank_positions", "alibi_slopes"):
        monkeypatch.setattr(oracle, name, replacement)
    with np.errstate(all="ignore"):
        assert not _pins_hold()
