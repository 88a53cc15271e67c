"""GPU parity of ra_rope (rotary position embedding, intelliparadigm.com
long-context survey §2.1.3) against the fp64 oracle, alone and followed by the
ring forward.

Tolerances: fp32 output within 4e-6 * max|x| of the exact rotation (angles are
reduced in double precision, the rotation runs in fp32); bf16 output within
half a bf16 ulp of the exact value plus the fp32 error (2^-8 |ref| + 2e-6
max|x|). The attention after RoPE keeps the bf16 attention tolerances, with the
oracle attending over its own rotation rounded to bf16 (the tensor the
attention consumes).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from ring_attention_ra_amd import _lib, configs, ring
from tests._cases import Case, draw, host64, log, max_abs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield
    torch.cuda.synchronize()


def _positions(length):
    rng = np.random.default_rng(7)
    fixed = np.array([0, 1, 2, 3, 63, 64, 4095, 131071, 1048575, 2 ** 30 - 1])
    return np.sort(np.unique(np.concatenate([fixed, rng.integers(0, 2 ** 30, length)])))[:length]


def _check(y, ref, x, dtype):
    err = np.abs(host64(y) - ref)
    xm = float(np.max(np.abs(host64(x)))) if x.numel() else 0.0
    if dtype == "fp32":
        bound = 4e-6 * xm
        ok = bool(np.all(err <= bound))
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 2e-6 * xm
        ok = bool(np.all(err <= bound))
    log(f"  max err {float(err.max()) if err.size else 0.0:.3g}")
    assert ok


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [128, 64, 6, 200])
@pytest.mark.parametrize("inplace", [False, True])
def test_rope_matches_oracle(dtype, d, inplace):
    length = 40
    pos = _positions(length)
    log(f"case rope {dtype} d={d} inplace={inplace}")
    x = si.normal((2, 3, length, d), si.seed_for(81, si.Q_STREAM), 1.0, dtype, "cuda")
    pos_t = torch.from_numpy(pos.astype(np.int32)).cuda()
    if inplace:
        y = x.clone()
        _lib.ra_rope(y, y, pos_t)
    else:
        y = torch.empty_like(x)
        _lib.ra_rope(x, y, pos_t)
    torch.cuda.synchronize()
    ref = oracle.rotary_embedding(host64(x), pos)
    _check(y, ref, x, dtype)


def test_rope_zero_positions_is_identity_bitwise():
    x = si.normal((1, 2, 33, 128), si.seed_for(82, si.Q_STREAM), 1.0, "bf16", "cuda")
    y = torch.empty_like(x)
    _lib.ra_rope(x, y, torch.zeros(33, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("layout", ["zigzag", "contiguous"])
def test_rope_then_ring_forward(layout):
    n = 4
    case = Case("bf16", 1, 4, 2, 128, n * 256, n, layout, True, False, seed=71)
    log(f"case rope + {case.tag()}")
    q, k, v = draw(case)
    r = n - 1
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, n, layout, r)
    # each chunk is turned by its tokens' global positions
    _lib.ra_rope(q_loc, q_loc, pos[r].contiguous())
    for s in range(n):
        _lib.ra_rope(k_ch[s], k_ch[s], pos[s].contiguous())
    o, lse = ring.forward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), None)
    torch.cuda.synchronize()
    g = np.arange(case.seq_len)
    to_bf16 = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    qr = to_bf16(oracle.rotary_embedding(host64(q), g))
    kr = to_bf16(oracle.rotary_embedding(host64(k), g))
    o_ref, lse_ref = oracle.attention_rank_share(qr, kr, host64(v), n, r, layout, True, case.sc(), None)
    eo, el = max_abs(host64(o), o_ref), max_abs(host64(lse), lse_ref)
    log(f"  max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    assert eo <= 2e-2 and el <= 1e-3


def test_rope_full_size_1m_query_chunk_sampled():
    """RoPE of the 1M-token zig-zag rank share's query chunk (positions up to
    2^20 - 1), checked on sampled rows of two heads."""
    w = configs.get(5)
    log(f"case rope {w.name} (query chunk, sampled)")
    pos = torch.empty((w.chunk,), dtype=torch.int32, device="cuda")
    _lib.ra_positions(w.seq_len, w.n_ranks, w.rank, w.layout, pos)
    x = si.normal((w.batch, w.heads_q, w.chunk, w.head_dim), si.seed_for(83, si.Q_STREAM), 1.0, "bf16", "cuda")
    y = torch.empty_like(x)
    _lib.ra_rope(x, y, pos)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(w.chunk - 4, w.chunk), rng.integers(0, w.chunk, 24)]))
    p = pos.cpu().numpy()[rows]
    assert p.max() == w.seq_len - 1 or rows.max() < w.chunk - 1
    for h in (0, w.heads_q - 1):
        xs = x[0, h, torch.from_numpy(rows).cuda()]
        ref = oracle.rotary_embedding(host64(xs), p)
        _check(y[0, h, torch.from_numpy(rows).cuda()], ref, xs, "bf16")
