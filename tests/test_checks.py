"""GPU tests of the optional checks: ra_count_nonfinite, RA_CHECK_FINITE=1 on
the compute entry points (a NaN planted in one K/V chunk, standing in for a
corrupted ring transfer, is refused before it reaches the state), and
RA_DEBUG=1 (position order). Expected counts come from numpy on host copies.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from ring_attention_ra_amd import _lib, ring
from tests._cases import Case, draw, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [1, 255, 4097, 1 << 20])
def test_count_nonfinite_matches_numpy(dtype, n):
    g = torch.Generator().manual_seed(n)
    x = torch.randn(n, generator=g).to(dtype)
    idx = torch.randint(0, n, (min(n, 7),), generator=g)
    specials = [float("nan"), float("inf"), -float("inf"), 3.0e38, -0.0, float("nan"), 1.0]
    for i, v in zip(idx.tolist(), specials):
        x[i] = v
    x[-1] = float("inf") if n > 3 else x[-1]  # the last element is counted too
    expect = int((~np.isfinite(x.float().numpy())).sum())
    got = _lib.ra_count_nonfinite(x.cuda())
    log(f"  n={n} {dtype}: {got} non-finite (expected {expect})")
    assert got == expect
    # a bf16 NaN with only a low mantissa bit set, and the largest finite value
    if dtype == torch.bfloat16:
        raw = np.array([0x7F81, 0x7F7F, 0xFF80, 0x0001], dtype=np.uint16).view(np.int16)
        y = torch.from_numpy(raw).view(torch.bfloat16)
        assert _lib.ra_count_nonfinite(y.cuda()) == 2


def _fold_all(case, r, q_loc, k_ch, v_ch, pos, slopes):
    st = ring.State(_lib.dims_of(q_loc, k_ch[0]), q_loc.device)
    for s in ring.ring_schedule(case.n_ranks, r):
        ring.fold(st, q_loc, k_ch[s], v_ch[s], pos[r], pos[s], case.causal, case.sc(), slopes)
    return st


def _state(st):
    torch.cuda.synchronize()
    return [t.cpu().numpy().tobytes() for t in (st.o_acc, st.m, st.l)]


@pytest.mark.parametrize("dtype,layout,alibi", [("bf16", "zigzag", True), ("fp32", "contiguous", False)])
def test_check_finite_refuses_a_corrupted_chunk(monkeypatch, dtype, layout, alibi):
    case = Case(dtype, 1, 2, 2, 128 if dtype == "bf16" else 64, 4 * 320, 4, layout, True, alibi, seed=71)
    log(f"case {case.tag()}")
    q, k, v = draw(case)
    r = 3
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
    slopes = ring.alibi_slopes(case.heads_q) if alibi else None
    plain = _state(_fold_all(case, r, q_loc, k_ch, v_ch, pos, slopes))

    monkeypatch.setenv("RA_CHECK_FINITE", "1")
    checked = _state(_fold_all(case, r, q_loc, k_ch, v_ch, pos, slopes))
    assert checked == plain, "the check changed the result"

    # One value of the chunk that arrives at hop 2 is corrupted.
    bad = (r - 2) % case.n_ranks
    k_bad = k_ch[bad].clone()
    k_bad[0, 1, 17, 5] = float("nan")
    st = ring.State(_lib.dims_of(q_loc, k_ch[0]), q.device)
    for j, s in enumerate(ring.ring_schedule(case.n_ranks, r)):
        kk = k_bad if s == bad else k_ch[s]
        if s == bad:
            before = _state(st)
            with pytest.raises(_lib.RaError) as e:
                ring.fold(st, q_loc, kk, v_ch[s], pos[r], pos[s], True, case.sc(), slopes)
            assert e.value.status == _lib.RA_ERR_NONFINITE and "k_blk" in str(e.value), str(e.value)
            log(f"  hop {j}: {e.value}")
            assert _state(st) == before, "a refused chunk must leave the state as it was"
            kk = k_ch[s]  # the chunk is sent again, intact
        ring.fold(st, q_loc, kk, v_ch[s], pos[r], pos[s], True, case.sc(), slopes)
    assert _state(st) == plain

    # Corrupted values: an Inf in V, and a NaN in the query chunk.
    v_bad = v_ch[0].clone()
    v_bad[0, 0, -1, -1] = float("inf")
    with pytest.raises(_lib.RaError) as e:
        ring.fold(st, q_loc, k_ch[0], v_bad, pos[r], pos[0], True, case.sc(), slopes)
    assert e.value.status == _lib.RA_ERR_NONFINITE and "v_blk" in str(e.value)
    q_bad = q_loc.clone()
    q_bad[0, 0, 0, 0] = float("nan")
    with pytest.raises(_lib.RaError) as e:
        ring.fold(st, q_bad, k_ch[0], v_ch[0], pos[r], pos[0], True, case.sc(), slopes)
    assert e.value.status == _lib.RA_ERR_NONFINITE and ": q holds" in str(e.value)


def test_check_finite_output_side_and_finalize(monkeypatch):
    """A state that was corrupted outside the library (NaN in o_acc) is caught
    after the next step; rows with no key (m = -inf, l = 0) are not errors."""
    monkeypatch.setenv("RA_CHECK_FINITE", "1")
    case = Case("bf16", 1, 2, 2, 128, 4 * 256, 4, "contiguous", True, False, seed=73)
    q, k, v = draw(case)
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, 4, "contiguous", 0)
    dims = _lib.dims_of(q_loc, k_ch[0])
    st = ring.State(dims, q.device)
    o, lse = ring.finalize(st, torch.bfloat16)  # every row empty: O = 0, LSE = -inf, allowed
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lse))
    ring.fold(st, q_loc, k_ch[1], v_ch[1], pos[0], pos[1], True, case.sc(), None)  # all masked: no-op
    st.o_acc[0, 1, 3, 7] = float("nan")
    with pytest.raises(_lib.RaError) as e:
        ring.fold(st, q_loc, k_ch[0], v_ch[0], pos[0], pos[0], True, case.sc(), None)
    assert e.value.status == _lib.RA_ERR_NONFINITE and "o_acc" in str(e.value) and "after" in str(e.value)
    with pytest.raises(_lib.RaError) as e:
        ring.finalize(st, torch.bfloat16)
    assert e.value.status == _lib.RA_ERR_NONFINITE and "o_acc" in str(e.value)


def test_check_finite_backward(monkeypatch):
    case = Case("bf16", 1, 2, 1, 128, 2 * 256, 2, "zigzag", True, True, seed=75)
    q, k, v, do = draw(case, with_do=True)
    r = 1
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
    sl = ring.alibi_slopes(case.heads_q)
    o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), sl)
    ref = [t.cpu() for t in ring.backward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), sl, o, lse, do)]
    monkeypatch.setenv("RA_CHECK_FINITE", "1")
    got = [t.cpu() for t in ring.backward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), sl, o, lse, do)]
    assert all(torch.equal(a, b) for a, b in zip(ref, got))
    do_bad = do.clone()
    do_bad[0, 1, 100, 64] = -float("inf")
    with pytest.raises(_lib.RaError) as e:
        ring.backward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), sl, o, lse, do_bad)
    assert e.value.status == _lib.RA_ERR_NONFINITE and "d_o" in str(e.value)
    lse_bad = lse.clone()
    lse_bad[0, 0, 3] = float("nan")
    dims = _lib.dims_of(q_loc, k_ch[0])
    delta = torch.zeros_like(lse)
    dq = torch.zeros(q_loc.shape, dtype=torch.float32, device=q.device)
    dk = torch.zeros(k_ch[0].shape, dtype=torch.float32, device=q.device)
    with pytest.raises(_lib.RaError) as e:
        _lib.ra_step_bwd(dims, q_loc, k_ch[0], v_ch[0], pos[r], pos[0], True, case.sc(), sl, do, lse_bad, delta,
                         dq, dk, torch.zeros_like(dk))
    assert e.value.status == _lib.RA_ERR_NONFINITE and "lse" in str(e.value)


def test_debug_checks_position_order(monkeypatch):
    case = Case("bf16", 1, 2, 2, 128, 2 * 256, 2, "zigzag", True, False, seed=77)
    q, k, v = draw(case)
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, 2, "zigzag", 1)
    st = ring.State(_lib.dims_of(q_loc, k_ch[0]), q.device)
    bad_order = pos[0].clone()
    bad_order[10], bad_order[11] = pos[0][11], pos[0][10]
    negative = pos[1].clone()
    negative[0] = -1
    # without RA_DEBUG the precondition is the caller's (nothing is checked)
    monkeypatch.setenv("RA_DEBUG", "1")
    ring.fold(st, q_loc, k_ch[0], v_ch[0], pos[1], pos[0], True, case.sc(), None)  # valid
    before = _state(st)
    for qp, kp, name in [(pos[1], bad_order, "k_pos"), (negative, pos[0], "q_pos")]:
        with pytest.raises(_lib.RaError) as e:
            ring.fold(st, q_loc, k_ch[0], v_ch[0], qp, kp, True, case.sc(), None)
        assert e.value.status == _lib.RA_ERR_INVALID_ARGUMENT and name in str(e.value), str(e.value)
    assert _state(st) == before
    repeated = pos[0].clone()
    repeated[5] = repeated[4]
    dims = _lib.dims_of(q_loc, k_ch[0])
    z = torch.zeros(q_loc.shape, dtype=torch.float32, device=q.device)
    zk = torch.zeros(k_ch[0].shape, dtype=torch.float32, device=q.device)
    lse = torch.zeros(q_loc.shape[:3], dtype=torch.float32, device=q.device)
    with pytest.raises(_lib.RaError) as e:
        _lib.ra_step_bwd(dims, q_loc, k_ch[0], v_ch[0], pos[1], repeated, True, case.sc(), None, q_loc, lse, lse,
                         z, zk, zk.clone())
    assert e.value.status == _lib.RA_ERR_INVALID_ARGUMENT and "k_pos" in str(e.value)
