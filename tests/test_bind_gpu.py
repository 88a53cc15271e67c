"""Bound calls (_lib.bind) issue exactly the calls of the plain binding: a
ring forward through bound calls, run twice, gives bitwise the outputs of the
same ring through the plain entry points."""

import pytest
import torch

from ring_attention_ra_amd import _lib, ring
from tests._cases import Case, draw, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("alibi", [False, True])
def test_bound_ring_matches_plain_ring(alibi):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = Case("bf16", 1, 4, 2, 128, 2 * 300, 2, "zigzag", True, alibi, seed=515)
    log(f"case {case.tag()}")
    q, k, v = draw(case)
    r = 1
    slopes = ring.alibi_slopes(case.heads_q) if alibi else None
    q_loc, k_ch, v_ch, pos = ring.shard(q, k, v, case.n_ranks, case.layout, r)
    o_ref, lse_ref = ring.forward(q_loc, k_ch, v_ch, pos, r, True, case.sc(), slopes)

    dims = _lib.dims_of(q_loc, k_ch[0])
    o_acc = torch.empty(q_loc.shape, dtype=torch.float32, device=q_loc.device)
    m = torch.empty(q_loc.shape[:-1], dtype=torch.float32, device=q_loc.device)
    l = torch.empty_like(m)
    o, lse = torch.empty_like(q_loc), torch.empty_like(m)
    calls = [_lib.bind(_lib.ra_state_init, dims, o_acc, m, l)]
    calls += [_lib.bind(_lib.ra_step_fwd, dims, q_loc, k_ch[s], v_ch[s], pos[r], pos[s], True, case.sc(), slopes,
                        o_acc, m, l) for s in ring.ring_schedule(case.n_ranks, r)]
    calls.append(_lib.bind(_lib.ra_finalize, dims, o_acc, m, l, o, lse))
    for rep in range(2):
        o.fill_(0)
        lse.fill_(0)
        for call in calls:
            call()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
