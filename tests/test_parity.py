"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (max abs error): fp32 1e-5 on O and LSE; bf16 inputs with fp32
accumulation 2e-2 on O and 1e-3 on LSE. Integer and data-movement work
(positions, layout permutation) is compared bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ring_attention_ra_amd import _lib, configs, ring
from tests._cases import Case, Timer, draw, host64, host_heads, log, max_abs, oracle_slopes, record

pytestmark = pytest.mark.gpu

TOL = {"fp32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()  # fails loudly when libra.so is missing
    yield
    torch.cuda.synchronize()


def _slopes_dev(case):
    return ring.alibi_slopes(case.heads_q) if case.alibi else None


def _run_gpu(case, ranks, q, k, v):
    """O, LSE of each rank (GPU), plus the positions the library produced."""
    out = {}
    for r in ranks:
        q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
        o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, case.causal, case.sc(), _slopes_dev(case))
        out[r] = (o, lse, pos)
    torch.cuda.synchronize()
    return out


def _check_full(case, ranks=None):
    log(f"case {case.tag()}")
    ranks = list(range(case.n_ranks)) if ranks is None else ranks
    q, k, v = draw(case)
    res = _run_gpu(case, ranks, q, k, v)
    qh, kh, vh = host64(q), host64(k), host64(v)
    tol_o, tol_l = TOL[case.dtype]
    for r in ranks:
        o_ref, lse_ref = oracle.attention_rank_share(qh, kh, vh, case.n_ranks, r, case.layout, case.causal,
                                                     case.sc(), oracle_slopes(case))
        o, lse, pos = res[r]
        assert np.array_equal(pos.cpu().numpy(), np.stack(
            [oracle.rank_positions(case.seq_len, case.n_ranks, i, case.layout) for i in range(case.n_ranks)]))
        eo, el = max_abs(host64(o), o_ref), max_abs(host64(lse), lse_ref)
        log(f"  rank {r}: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
        record(case.tag(), r, {"max_abs_O": eo, "max_abs_LSE": el})
        assert eo <= tol_o and el <= tol_l, (r, eo, el)


# ---------------------------------------------------------------------------
# positions and permutation: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("s,n", [(256, 4), (16384, 8), (96, 3), (64, 64)])
def test_positions_bitwise(layout, s, n):
    allr = ring.positions(s, n, layout).cpu().numpy()
    ref = np.stack([oracle.rank_positions(s, n, r, layout) for r in range(n)])
    assert np.array_equal(allr, ref)
    for r in (0, n - 1):
        assert np.array_equal(ring.positions(s, n, layout, rank=r).cpu().numpy(), ref[r])


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("dtype,shape,n", [
    (torch.bfloat16, (2, 3, 48, 8), 4),
    (torch.bfloat16, (1, 2, 64, 128), 8),
    (torch.float32, (1, 4, 96, 1), 3),      # LSE-like rows of one fp32
    (torch.bfloat16, (2, 2, 40, 3), 5),     # 6-byte rows: 2-byte copy units
    (torch.float32, (1, 1, 256, 64), 4),
])
def test_permute_bitwise(layout, dtype, shape, n):
    b, h, s, d = shape
    x = torch.randn(shape, generator=torch.Generator().manual_seed(5)).to(dtype).cuda()
    xr = oracle.permute_to_ranks(x.float().cpu().numpy(), n, layout)
    y = torch.empty((n, b, h, s // n, d), dtype=dtype, device="cuda")
    pos = torch.empty((n, s // n), dtype=torch.int32, device="cuda")
    _lib.ra_layout_permute(x, y, pos, b * h, s, d, n, layout, rank=-1)
    assert np.array_equal(y.float().cpu().numpy(), xr)
    back = torch.empty_like(x)
    _lib.ra_layout_permute(y, back, None, b * h, s, d, n, layout, rank=-1, inverse=1)
    assert torch.equal(back.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    for r in (0, n - 1):
        yr = torch.empty((b, h, s // n, d), dtype=dtype, device="cuda")
        _lib.ra_layout_permute(x, yr, None, b * h, s, d, n, layout, rank=r)
        assert np.array_equal(yr.float().cpu().numpy(), xr[r])
        part = torch.zeros_like(x)
        _lib.ra_layout_permute(yr, part, None, b * h, s, d, n, layout, rank=r, inverse=1)
        p = oracle.rank_positions(s, n, r, layout)
        ref = np.zeros(shape, dtype=np.float32)
        ref[:, :, p] = xr[r]
        assert np.array_equal(part.float().cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# forward parity
# ---------------------------------------------------------------------------

def test_workload_fp32_rank_share_all_ranks():
    w = configs.get(1)
    case = Case("fp32", w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_len, w.n_ranks, w.layout,
                seed=w.index)
    _check_full(case)


@pytest.mark.parametrize("d", [3, 33, 64, 100, 128])
@pytest.mark.parametrize("layout,causal,alibi,hq,hkv", [
    ("zigzag", True, False, 2, 2),
    ("contiguous", True, True, 4, 2),
    ("zigzag", False, True, 2, 1),
])
def test_fwd_fp32_variants(d, layout, causal, alibi, hq, hkv):
    _check_full(Case("fp32", 2, hq, hkv, d, 4 * 76, 4, layout, causal, alibi, seed=11))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout,causal,alibi,hq,hkv,n,c", [
    ("zigzag", True, False, 2, 2, 4, 320),       # 3 query tiles (last ragged), 5 key tiles
    ("contiguous", True, False, 2, 1, 4, 300),   # ragged query and key tiles, GQA
    ("zigzag", True, True, 4, 2, 2, 384),        # ALiBi + GQA
    ("contiguous", True, True, 2, 2, 3, 200),
    ("zigzag", False, False, 2, 2, 2, 256),
    ("contiguous", False, True, 2, 1, 2, 150),
])
def test_fwd_bf16_variants(d, layout, causal, alibi, hq, hkv, n, c):
    _check_full(Case("bf16", 1, hq, hkv, d, n * c, n, layout, causal, alibi, seed=21))


@pytest.mark.parametrize("layout,causal,alibi,hq,hkv,n,c,ranks", [
    ("zigzag", True, False, 2, 2, 4, 40, None),          # chunk shorter than one 64-key tile
    ("contiguous", True, False, 1, 1, 2, 4497, None),    # 71 key tiles, ragged
    ("zigzag", True, False, 2, 2, 2, 4497, None),
    ("zigzag", True, True, 2, 1, 2, 4497, None),         # ALiBi + GQA over the same range
    # chunks longer than any workload's (258 key tiles), ragged
    ("contiguous", True, False, 1, 1, 2, 16500, [1]),
    ("zigzag", True, False, 1, 1, 2, 16500, [1]),
])
def test_fwd_bf16_tile_range_edges(layout, causal, alibi, hq, hkv, n, c, ranks):
    _check_full(Case("bf16", 1, hq, hkv, 128, n * c, n, layout, causal, alibi, seed=25), ranks=ranks)


# The persistent bf16 launch: with fewer query tiles than CUs each work-group
# takes one tile; with more (the second and third cases on a 256-CU GPU) each
# walks several, heaviest and lightest in turn (ragged ends, GQA, more than 64
# key tiles).
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("hq,hkv,n,c", [(2, 1, 2, 4497), (132, 66, 2, 300), (16, 8, 2, 4497)])
def test_fwd_bf16_one_and_several_tiles_per_work_group(d, layout, hq, hkv, n, c):
    _check_full(Case("bf16", 1, hq, hkv, d, n * c, n, layout, True, False, seed=29), ranks=[n - 1])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("scale", [0.0, -0.06])
def test_fwd_scale_zero_and_negative_with_alibi(dtype, scale):
    # With scale <= 0 the fast paths that rely on scale > 0 are not taken.
    _check_full(Case(dtype, 1, 4, 2, 128 if dtype == "bf16" else 64, 3 * 320, 3, "zigzag", True, True, seed=27,
                     scale=scale))


def test_fwd_bf16_batch2_and_std():
    _check_full(Case("bf16", 2, 3, 1, 128, 4 * 256, 4, "zigzag", True, True, std=0.7, seed=23))


def test_state_after_partial_ring():
    case = Case("bf16", 1, 4, 2, 128, 4 * 256, 4, "zigzag", True, True, seed=31)
    q, k, v = draw(case)
    qh, kh, vh = host64(q), host64(k), host64(v)
    r = 1
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
    sched = ring.ring_schedule(case.n_ranks, r)
    state = ring.State(_lib.dims_of(q_loc, k_ch[0]), q.device)
    for j, s in enumerate(sched):
        ring.fold(state, q_loc, k_ch[s], v_ch[s], pos[r], pos[s], True, case.sc(), _slopes_dev(case))
        torch.cuda.synchronize()
        o_acc, m, l = oracle.accumulator_state(qh, kh, vh, case.n_ranks, r, case.layout, True, case.sc(),
                                               oracle_slopes(case), key_chunks=sched[:j + 1])
        o_ref, lse_ref = oracle.finalize_state(o_acc, m, l)
        o, lse = ring.finalize(state, torch.bfloat16)
        # The bf16 kernel keeps m as the reference of its exponentials: at most
        # the row max and less by no more than 14 ln 2 (the bound its lazy
        # rescale keeps), with l and o_acc taken against it, so m + ln l is
        # the log-sum-exp and o_acc / l the output whatever m is.
        sm, sl, so = host64(state.m), host64(state.l), host64(state.o_acc)
        seen = np.isfinite(m)
        gap = m[seen] - sm[seen]
        s_o, s_lse = oracle.finalize_state(so, sm, sl)
        eo = max_abs(host64(o), o_ref)
        el = max_abs(host64(lse), lse_ref)
        es_l = max_abs(s_lse[seen], lse_ref[seen])
        es_o = max_abs(s_o, o_ref)
        log(f"  after {j + 1} chunks: m gap in [{gap.min():.3g}, {gap.max():.3g}] max|dO|={eo:.3g} "
            f"max|dLSE|={el:.3g} state: max|dLSE|={es_l:.3g} max|dO|={es_o:.3g}")
        assert gap.min() >= -1e-3 and gap.max() <= 14 * np.log(2.0) + 1e-3
        assert np.all(sl[seen] >= 1.0 - 1e-3)
        assert eo <= 2e-2 and el <= 1e-3 and es_l <= 1e-3 and es_o <= 2e-2
        # empty rows keep the start state exactly
        empty = np.isneginf(m)
        assert np.all(np.isneginf(host64(state.m)[empty])) and np.all(host64(state.l)[empty] == 0)


def test_workload_16k_zigzag_all_ranks_full():
    w = configs.get(2)
    case = Case("bf16", w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_len, w.n_ranks, w.layout,
                seed=w.index)
    _check_full(case)


def _sampled_full_size(w, n_rows=48, heads=None, rank=None):
    """Full-size run of a workload (the benchmark's launch configuration) for
    one rank (the workload's own by default); the oracle recomputes a sample
    of rows and heads one by one."""
    rank = w.rank if rank is None else rank
    case = Case(w.dtype, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_len, w.n_ranks, w.layout,
                w.causal, w.alibi, w.std, seed=w.index)
    log(f"case {w.name} rank {rank} (sampled)")
    with Timer("draw + GPU ring"):
        q, k, v = draw(case)
        res = _run_gpu(case, [rank], q, k, v)
    o, lse, _ = res[rank]
    c = w.chunk
    rng = np.random.default_rng(w.index)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(c - 16, c), rng.integers(0, c, n_rows - 32)]))
    if heads is None:
        heads = sorted({0, w.heads_q - 1, int(rng.integers(w.heads_q))})
    g = w.heads_q // w.heads_kv
    with Timer("host copies"):
        qh = host_heads(q, heads)
        kh = host_heads(k, [h // g for h in heads])
        vh = host_heads(v, [h // g for h in heads])
    with Timer("oracle"):
        o_ref, lse_ref = oracle.attention_rank_share(qh, kh, vh, w.n_ranks, rank, w.layout, w.causal, w.scale,
                                                     oracle_slopes(case), rows=rows, heads=heads)
    o_g = host64(o[:, heads][:, :, rows])
    l_g = host64(lse[:, heads][:, :, rows])
    eo, el = max_abs(o_g, o_ref), max_abs(l_g, lse_ref)
    log(f"  rows={rows.size} heads={heads}: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    record(w.name, rank, {"max_abs_O": eo, "max_abs_LSE": el}, sample=f"{rows.size} rows x heads {heads}")
    tol_o, tol_l = TOL[w.dtype]
    assert eo <= tol_o and el <= tol_l
    # a property that holds at any size: every output is finite
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("rank", [0, 7])
def test_workload_128k_zigzag_sampled(rank):
    _sampled_full_size(configs.get(3), rank=rank)


@pytest.mark.parametrize("rank", [0, 3])
def test_workload_64k_gqa_alibi_sampled(rank):
    _sampled_full_size(configs.get(4), rank=rank)


@pytest.mark.parametrize("rank", [0, 63])
def test_workload_1m_zigzag_forward_sampled(rank):
    # Under zig-zag, rank 0's first row (position 0) sees no key in any chunk
    # but its own: every later step has a row with no visible key.
    _sampled_full_size(configs.get(5), heads=[0, 15], rank=rank)


# ---------------------------------------------------------------------------
# semantics of the step interface
# ---------------------------------------------------------------------------

def _state_bytes(state):
    torch.cuda.synchronize()
    return (state.o_acc.cpu().numpy().tobytes(), state.m.cpu().numpy().tobytes(),
            state.l.cpu().numpy().tobytes())


def test_deterministic_and_resumable():
    case = Case("bf16", 1, 4, 4, 128, 8 * 256, 8, "zigzag", True, False, seed=41)
    q, k, v = draw(case)
    r = 5
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
    sched = ring.ring_schedule(case.n_ranks, r)
    dims = _lib.dims_of(q_loc, k_ch[0])

    def run(resume_at=None):
        st = ring.State(dims, q.device)
        for j, s in enumerate(sched):
            if j == resume_at:
                saved = [t.cpu() for t in (st.o_acc, st.m, st.l)]
                st = ring.State(dims, q.device)
                for dst, src in zip((st.o_acc, st.m, st.l), saved):
                    dst.copy_(src)
            ring.fold(st, q_loc, k_ch[s], v_ch[s], pos[r], pos[s], True, case.sc(), None)
        return _state_bytes(st)

    a, b, c = run(), run(), run(resume_at=3)
    assert a == b, "two runs differ"
    assert a == c, "resumed run differs"


def test_masked_chunk_and_empty_inputs_leave_state_unchanged():
    case = Case("bf16", 1, 2, 2, 128, 4 * 256, 4, "contiguous", True, False, seed=51)
    q, k, v = draw(case)
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, 4, "contiguous", 0)
    dims = _lib.dims_of(q_loc, k_ch[0])
    st = ring.State(dims, q.device)
    ring.fold(st, q_loc, k_ch[0], v_ch[0], pos[0], pos[0], True, case.sc(), None)
    before = _state_bytes(st)
    for s in (1, 2, 3):  # later chunks are entirely in the causal future of rank 0
        ring.fold(st, q_loc, k_ch[s], v_ch[s], pos[0], pos[s], True, case.sc(), None)
    assert _state_bytes(st) == before
    # a zero-length chunk and a zero-length query block enqueue nothing
    empty_dims = _lib.make_dims(1, 2, 2, 128, 256, 0, torch.bfloat16)
    assert _lib.lib().ra_step_fwd(empty_dims, None, None, None, None, None, 1, 0.1, None, None, None, None,
                                  None) == 0
    assert _state_bytes(st) == before


def test_fp32_finalize_of_unvisited_rows():
    dims = _lib.make_dims(1, 1, 1, 64, 10, 10, torch.float32)
    st = ring.State(dims, torch.device("cuda"))
    o, lse = ring.finalize(st, torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


# ---------------------------------------------------------------------------
# backward parity: bf16 (D = 128) max |g - g_ref| <= 1e-2 * max |g_ref|;
# fp32 max |g - g_ref| <= 1e-5 * max(1, max |g_ref|)
# ---------------------------------------------------------------------------

BWD_REL = 1e-2


def _bwd_gpu(case, r, q, k, v, do):
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
    sl = _slopes_dev(case)
    o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, case.causal, case.sc(), sl)
    dq, dk, dv = ring.backward(q_loc, k_ch, v_ch, pos, r, case.causal, case.sc(), sl, o, lse, do)
    torch.cuda.synchronize()
    return dq, dk, dv


def _rel_err(got, ref):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    return max_abs(got, ref) / max(scale, 1e-30)


@pytest.mark.parametrize("layout,causal,alibi,hq,hkv,n,c", [
    ("zigzag", True, False, 2, 2, 4, 256),
    ("contiguous", True, False, 4, 2, 4, 192),     # GQA, ragged tiles
    ("zigzag", True, True, 2, 1, 2, 320),          # ALiBi + GQA, ragged
    ("contiguous", False, False, 2, 2, 2, 200),    # no mask, ragged
    ("contiguous", True, True, 2, 2, 3, 128),
    ("zigzag", True, False, 8, 2, 2, 64),          # 64-key chunk: two idle key blocks, one tile per head
    ("contiguous", False, True, 4, 4, 1, 96),      # one rank, ALiBi without the causal mask
])
def test_bwd_variants(layout, causal, alibi, hq, hkv, n, c):
    case = Case("bf16", 1, hq, hkv, 128, n * c, n, layout, causal, alibi, seed=61)
    log(f"case {case.tag()}")
    q, k, v, do = draw(case, with_do=True)
    qh, kh, vh = host64(q), host64(k), host64(v)
    for r in sorted({0, n - 1}):
        dq, dk, dv = _bwd_gpu(case, r, q, k, v, do)
        dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, host64(do), n, r, layout, causal, case.sc(),
                                                           oracle_slopes(case))
        e_q = _rel_err(host64(dq), dq_r)
        e_k = _rel_err(host64(dk), oracle.permute_to_ranks(dk_r, n, layout))
        e_v = _rel_err(host64(dv), oracle.permute_to_ranks(dv_r, n, layout))
        log(f"  rank {r}: rel dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g}")
        record(case.tag(), r, {"rel_dQ": e_q, "rel_dK": e_k, "rel_dV": e_v})
        assert e_q <= BWD_REL and e_k <= BWD_REL and e_v <= BWD_REL


@pytest.mark.parametrize("layout,alibi,hq,hkv,n,c,ranks", [
    # 16K zig-zag over 8 chunks of 2048: a key's dK / dV sums over up to 2048
    # rows of the rank's chunk, every row and key compared.
    ("zigzag", False, 2, 2, 8, 2048, (0, 7)),
    # contiguous GQA 8/2 + ALiBi: the last rank's keys of chunk 0 are summed over
    # all 2048 rows of each of the 4 query heads that share their K/V head.
    ("contiguous", True, 8, 2, 4, 2048, (0, 3)),
    # one 16384-row chunk attending to itself: the dK / dV of key 0 is a sum
    # over all 16384 rows, the length of a full-size chunk.
    ("contiguous", False, 1, 1, 1, 16384, (0,)),
    # 176 query heads over 22 K/V heads, ragged chunks of 300: 528 query tiles
    # of 128 rows, more than the persistent dQ launch has work-groups on a
    # 256-CU GPU, so each walks several (both layouts, with and without ALiBi).
    ("zigzag", False, 176, 22, 2, 300, (1,)),
    ("contiguous", True, 176, 22, 2, 300, (1,)),
])
def test_bwd_long_sums_full(layout, alibi, hq, hkv, n, c, ranks):
    case = Case("bf16", 1, hq, hkv, 128, n * c, n, layout, True, alibi, seed=65)
    log(f"case {case.tag()}")
    q, k, v, do = draw(case, with_do=True)
    qh, kh, vh = host64(q), host64(k), host64(v)
    for r in ranks:
        with Timer(f"rank {r} GPU"):
            dq, dk, dv = _bwd_gpu(case, r, q, k, v, do)
        with Timer(f"rank {r} oracle"):
            dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, host64(do), n, r, layout, True,
                                                               case.sc(), oracle_slopes(case))
        e_q = _rel_err(host64(dq), dq_r)
        e_k = _rel_err(host64(dk), oracle.permute_to_ranks(dk_r, n, layout))
        e_v = _rel_err(host64(dv), oracle.permute_to_ranks(dv_r, n, layout))
        log(f"  rank {r}: rel dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g}")
        record(case.tag(), r, {"rel_dQ": e_q, "rel_dK": e_k, "rel_dV": e_v})
        assert e_q <= BWD_REL and e_k <= BWD_REL and e_v <= BWD_REL


@pytest.mark.parametrize("scale", [0.0, -0.06])
def test_bwd_scale_zero_and_negative_with_alibi(scale):
    # The linear form of the ALiBi term divides by the scale; scale <= 0 takes
    # the per-element path.
    case = Case("bf16", 1, 4, 2, 128, 2 * 320, 2, "zigzag", True, True, seed=67, scale=scale)
    log(f"case {case.tag()} scale={scale}")
    q, k, v, do = draw(case, with_do=True)
    qh, kh, vh = host64(q), host64(k), host64(v)
    for r in (0, 1):
        dq, dk, dv = _bwd_gpu(case, r, q, k, v, do)
        dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, host64(do), 2, r, "zigzag", True, scale,
                                                           oracle_slopes(case))
        e_q = _rel_err(host64(dq), dq_r)
        e_k = _rel_err(host64(dk), oracle.permute_to_ranks(dk_r, 2, "zigzag"))
        e_v = _rel_err(host64(dv), oracle.permute_to_ranks(dv_r, 2, "zigzag"))
        log(f"  rank {r}: rel dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g}")
        assert np.isfinite(e_q) and e_q <= BWD_REL and e_k <= BWD_REL and e_v <= BWD_REL


def _abs_err_scaled(got, ref):
    return max_abs(got, ref) / max(1.0, float(np.max(np.abs(ref))) if ref.size else 0.0)


BWD_FP32 = 1e-5  # max |g - g_ref| <= 1e-5 * max(1, max |g_ref|)


@pytest.mark.parametrize("layout,causal,alibi,hq,hkv,d,n,c", [
    ("contiguous", True, False, 1, 1, 64, 4, 64),     # the fp32 workload's shape, every rank
    ("zigzag", True, True, 4, 2, 33, 3, 70),          # ALiBi + GQA, ragged D and lengths
    ("contiguous", False, True, 2, 1, 100, 2, 45),    # no mask
    ("zigzag", True, False, 2, 2, 128, 2, 96),
])
def test_bwd_fp32(layout, causal, alibi, hq, hkv, d, n, c):
    case = Case("fp32", 1, hq, hkv, d, n * c, n, layout, causal, alibi, seed=69)
    log(f"case {case.tag()}")
    q, k, v, do = draw(case, with_do=True)
    qh, kh, vh = host64(q), host64(k), host64(v)
    for r in range(n):
        dq, dk, dv = _bwd_gpu(case, r, q, k, v, do)
        dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, host64(do), n, r, layout, causal, case.sc(),
                                                           oracle_slopes(case))
        e_q = _abs_err_scaled(host64(dq), dq_r)
        e_k = _abs_err_scaled(host64(dk), oracle.permute_to_ranks(dk_r, n, layout))
        e_v = _abs_err_scaled(host64(dv), oracle.permute_to_ranks(dv_r, n, layout))
        log(f"  rank {r}: dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g} (x max(1, max|g|))")
        record(case.tag(), r, {"scaled_dQ": e_q, "scaled_dK": e_k, "scaled_dV": e_v})
        assert e_q <= BWD_FP32 and e_k <= BWD_FP32 and e_v <= BWD_FP32


def test_bwd_deterministic():
    case = Case("bf16", 1, 2, 2, 128, 4 * 256, 4, "zigzag", True, False, seed=63)
    q, k, v, do = draw(case, with_do=True)
    a = [t.cpu().numpy().tobytes() for t in _bwd_gpu(case, 3, q, k, v, do)]
    b = [t.cpu().numpy().tobytes() for t in _bwd_gpu(case, 3, q, k, v, do)]
    assert a == b


def test_workload_gqa_alibi_contiguous_backward_sampled():
    """Full-size forward + backward of the 64K GQA 64/8 + ALiBi contiguous share
    (rank 3); the oracle recomputes, for one key/value head and its eight query
    heads, dQ on sampled rows and dK, dV on sampled keys near the end of the
    sequence (seen by few rows under the causal mask)."""
    w = configs.get(6)
    case = Case(w.dtype, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_len, w.n_ranks, w.layout,
                w.causal, w.alibi, w.std, seed=w.index)
    log(f"case {w.name} (backward, sampled)")
    with Timer("draw + GPU forward/backward"):
        q, k, v, do = draw(case, with_do=True)
        dq, dk, dv = _bwd_gpu(case, w.rank, q, k, v, do)
    g = w.heads_q // w.heads_kv
    kv_heads = [5]
    qheads = [hk * g + i for hk in kv_heads for i in range(g)]
    c, n, s = w.chunk, w.n_ranks, w.seq_len
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(6), np.arange(c - 6, c), rng.integers(0, c, 12)]))
    keys = np.unique(np.concatenate([np.arange(s - 16, s), rng.integers(s - 96, s, 6)]))
    with Timer("host copies"):
        qh, kh, vh = host_heads(q, qheads), host_heads(k, kv_heads), host_heads(v, kv_heads)
        doh = do.float().cpu().numpy()
    with Timer("oracle"):
        dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, doh, n, w.rank, w.layout, w.causal,
                                                           w.scale, oracle_slopes(case), rows=rows, keys=keys,
                                                           kv_heads=kv_heads)
    owner = oracle.owner_rank(keys, s, n, w.layout)
    local = keys // n if w.layout == "zigzag" else keys % c
    hsel = torch.tensor(kv_heads, device=dk.device)
    dk_g = np.stack([host64(dk[int(owner[i])].index_select(1, hsel)[:, :, int(local[i])])
                     for i in range(keys.size)], axis=2)
    dv_g = np.stack([host64(dv[int(owner[i])].index_select(1, hsel)[:, :, int(local[i])])
                     for i in range(keys.size)], axis=2)
    dq_g = host64(dq[:, qheads][:, :, rows])
    e_q, e_k, e_v = _rel_err(dq_g, dq_r), _rel_err(dk_g, dk_r), _rel_err(dv_g, dv_r)
    log(f"  rows={rows.size} keys={keys.size}: rel dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g}")
    record(w.name, w.rank, {"rel_dQ": e_q, "rel_dK": e_k, "rel_dV": e_v},
           sample=f"{rows.size} rows, {keys.size} keys")
    assert e_q <= BWD_REL and e_k <= BWD_REL and e_v <= BWD_REL
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_workload_1m_zigzag_backward_sampled():
    """Full-size forward + backward of the 1M-token zig-zag share; the oracle
    recomputes dQ on sampled rows and dK, dV on sampled late keys (few rows see
    them under the causal mask) for two heads."""
    w = configs.get(5)
    case = Case(w.dtype, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_len, w.n_ranks, w.layout,
                w.causal, w.alibi, w.std, seed=w.index)
    log(f"case {w.name} (backward, sampled)")
    with Timer("draw + GPU forward/backward"):
        q, k, v, do = draw(case, with_do=True)
        dq, dk, dv = _bwd_gpu(case, w.rank, q, k, v, do)
    heads = [0, w.heads_q - 1]
    c, n, s = w.chunk, w.n_ranks, w.seq_len
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(c - 8, c), rng.integers(0, c, 16)]))
    keys = np.unique(np.concatenate([np.arange(s - 24, s), rng.integers(s - 4096, s, 8)]))
    with Timer("host copies"):
        qh, kh, vh = host_heads(q, heads), host_heads(k, heads), host_heads(v, heads)
        doh = do.float().cpu().numpy()
    with Timer("oracle"):
        dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, doh, n, w.rank, w.layout, w.causal,
                                                           w.scale, None, rows=rows, keys=keys, kv_heads=heads)
    owner = oracle.owner_rank(keys, s, n, w.layout)
    local = keys // n if w.layout == "zigzag" else keys % c
    hsel = torch.tensor(heads, device=dk.device)
    dk_g = np.stack([host64(dk[int(owner[i])].index_select(1, hsel)[:, :, int(local[i])])
                     for i in range(keys.size)], axis=2)
    dv_g = np.stack([host64(dv[int(owner[i])].index_select(1, hsel)[:, :, int(local[i])])
                     for i in range(keys.size)], axis=2)
    dq_g = host64(dq[:, heads][:, :, rows])
    e_q, e_k, e_v = _rel_err(dq_g, dq_r), _rel_err(dk_g, dk_r), _rel_err(dv_g, dv_r)
    log(f"  rows={rows.size} keys={keys.size}: rel dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g}")
    record(w.name, w.rank, {"rel_dQ": e_q, "rel_dK": e_k, "rel_dV": e_v},
           sample=f"{rows.size} rows, {keys.size} keys")
    assert e_q <= BWD_REL and e_k <= BWD_REL and e_v <= BWD_REL
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
