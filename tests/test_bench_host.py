"""Host logic of bench.py (no GPU): the FLOP accounting it reports and its
refusal of more than one GPU."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
from ring_attention_ra_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _positions(w):
    return torch.from_numpy(np.stack([oracle.rank_positions(w.seq_len, w.n_ranks, r, w.layout)
                                      for r in range(w.n_ranks)]).astype(np.int32))


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_visible_pairs_match_the_closed_forms(index):
    # Pairs per head for rank r: contiguous r*C^2 + C(C+1)/2, zig-zag N*C(C-1)/2 + C(r+1).
    w = configs.get(index)
    c, n, r = w.chunk, w.n_ranks, w.rank
    per_step = bench.visible_pairs_per_chunk(w, _positions(w))
    assert len(per_step) == n
    closed = r * c * c + c * (c + 1) // 2 if w.layout == "contiguous" else n * c * (c - 1) // 2 + c * (r + 1)
    assert sum(per_step) == closed
    assert sum(per_step) == oracle.visible_pairs(w.seq_len, n, r, w.layout, w.causal)
    # the step order is the ring's: own chunk first, and it holds the diagonal
    assert per_step[0] == c * (c + 1) // 2


def test_headline_flop_count():
    w = configs.HEADLINE
    pairs = sum(bench.visible_pairs_per_chunk(w, _positions(w)))
    assert pairs == 1073807360
    flop = 4.0 * w.head_dim * w.heads_q * w.batch * pairs
    assert flop == pytest.approx(1.759326e13, rel=1e-6)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "ONE GPU" in res.stderr
    assert res.stdout == ""
