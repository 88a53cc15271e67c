"""Seeded random sweep of small shapes: the HIP path (forward and backward,
bf16 and fp32) against the fp64 oracle, over batch, GQA group sizes, head
dims, ragged chunk lengths down to a single token, ring sizes from one rank, both
layouts, with and without the causal mask and ALiBi. Tolerances as in the
other parity tests: forward fp32 1e-5 on O and LSE, bf16 2e-2 on O and 1e-3 on
LSE; backward bf16 max |g - g_ref| <= 1e-2 max |g_ref| and fp32
max |g - g_ref| <= 1e-5 max(1, max |g_ref|)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ring_attention_ra_amd import _lib, ring
from tests._cases import Case, draw, host64, log, max_abs, oracle_slopes, record

pytestmark = pytest.mark.gpu

TOL = {"fp32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield
    torch.cuda.synchronize()


def _random_case(rng, dtype, backward, seed):
    b = int(rng.integers(1, 3))
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4]))
    n = int(rng.integers(1, 6))
    c = int(rng.integers(8 if backward else 1, 301))
    if dtype == "bf16":
        d = 128 if backward else int(rng.choice([64, 128]))
    else:
        d = int(rng.integers(1, 129))
    layout = str(rng.choice(["contiguous", "zigzag"]))
    causal = bool(rng.integers(0, 4) > 0)
    alibi = bool(rng.integers(0, 2))
    std = float(rng.choice([0.5, 0.7071067811865476, 1.0]))
    return Case(dtype, b, hkv * g, hkv, d, n * c, n, layout, causal, alibi, std, seed=seed)


def _ranks(rng, n):
    return sorted({n - 1, int(rng.integers(0, n))})


FWD_CASES = [(dtype, i) for dtype in ("bf16", "fp32") for i in range(24)]
BWD_CASES = [(dtype, i) for dtype in ("bf16", "fp32") for i in range(12)]


@pytest.mark.parametrize("dtype,i", FWD_CASES)
def test_forward_sweep(dtype, i):
    rng = np.random.default_rng(9000 + 100 * (dtype == "fp32") + i)
    case = _random_case(rng, dtype, False, seed=300 + i)
    log(f"case {case.tag()} std={case.std}")
    q, k, v = draw(case)
    qh, kh, vh = host64(q), host64(k), host64(v)
    slopes = ring.alibi_slopes(case.heads_q) if case.alibi else None
    tol_o, tol_l = TOL[dtype]
    for r in _ranks(rng, case.n_ranks):
        q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
        o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, case.causal, case.sc(), slopes)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_rank_share(qh, kh, vh, case.n_ranks, r, case.layout, case.causal,
                                                     case.sc(), oracle_slopes(case))
        eo, el = max_abs(host64(o), o_ref), max_abs(host64(lse), lse_ref)
        log(f"  rank {r}: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
        record(case.tag(), r, {"max_abs_O": eo, "max_abs_LSE": el}, sample="sweep")
        assert eo <= tol_o and el <= tol_l, (r, eo, el)


@pytest.mark.parametrize("dtype,i", BWD_CASES)
def test_backward_sweep(dtype, i):
    rng = np.random.default_rng(9500 + 100 * (dtype == "fp32") + i)
    case = _random_case(rng, dtype, True, seed=400 + i)
    log(f"case {case.tag()} std={case.std}")
    q, k, v, do = draw(case, with_do=True)
    qh, kh, vh, doh = host64(q), host64(k), host64(v), host64(do)
    slopes = ring.alibi_slopes(case.heads_q) if case.alibi else None
    for r in _ranks(rng, case.n_ranks):
        q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
        o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, case.causal, case.sc(), slopes)
        dq, dk, dv = ring.backward(q_loc, k_ch, v_ch, pos, r, case.causal, case.sc(), slopes, o, lse, do)
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = oracle.attention_rank_share_bwd(qh, kh, vh, doh, case.n_ranks, r, case.layout,
                                                           case.causal, case.sc(), oracle_slopes(case))
        pairs = ((host64(dq), dq_r), (host64(dk), oracle.permute_to_ranks(dk_r, case.n_ranks, case.layout)),
                 (host64(dv), oracle.permute_to_ranks(dv_r, case.n_ranks, case.layout)))
        errs = []
        for got, ref in pairs:
            m = float(np.max(np.abs(ref))) if ref.size else 0.0
            errs.append(max_abs(got, ref) / (max(m, 1e-30) if dtype == "bf16" else max(1.0, m)))
        log(f"  rank {r}: dQ={errs[0]:.3g} dK={errs[1]:.3g} dV={errs[2]:.3g}")
        record(case.tag(), r, {"sweep_dQ": errs[0], "sweep_dK": errs[1], "sweep_dV": errs[2]}, sample="sweep")
        tol = 1e-2 if dtype == "bf16" else 1e-5
        assert max(errs) <= tol, (r, errs)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 40)])
@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_forward_one_token_chunks(dtype, d, layout):
    # Chunks of a single token: every step is one key against one query.
    case = Case(dtype, 1, 4, 2, d, 5, 5, layout, True, True, seed=470)
    log(f"case {case.tag()}")
    q, k, v = draw(case)
    qh, kh, vh = host64(q), host64(k), host64(v)
    slopes = ring.alibi_slopes(case.heads_q)
    tol_o, tol_l = TOL[dtype]
    for r in range(case.n_ranks):
        q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
        o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), slopes)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_rank_share(qh, kh, vh, case.n_ranks, r, layout, True, case.sc(),
                                                     oracle_slopes(case))
        eo, el = max_abs(host64(o), o_ref), max_abs(host64(lse), lse_ref)
        log(f"  rank {r}: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
        assert eo <= tol_o and el <= tol_l, (r, eo, el)
