"""The workloads of the ring-attention step, by name and shape.

Each is one rank's share of a causal ring: a query chunk of C = S / N tokens
attending to the N K/V chunks it receives around the ring. Inputs are
synthetic, drawn by ``seeded_inputs`` with seed ``1000 * index + stream``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    dtype: str           # "fp32" or "bf16": dtype of Q, K, V, O
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_len: int
    n_ranks: int
    layout: str          # "contiguous" or "zigzag"
    rank: int            # the rank whose share is computed
    causal: bool = True
    alibi: bool = False
    std: float = 1.0     # inputs ~ N(0, std^2)
    backward: bool = False

    @property
    def chunk(self) -> int:
        return self.seq_len // self.n_ranks

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def describe(self) -> dict:
        return {"workload": self.name, "dtype": self.dtype, "batch": self.batch,
                "heads_q": self.heads_q, "heads_kv": self.heads_kv, "head_dim": self.head_dim,
                "seq_len": self.seq_len, "n_ranks": self.n_ranks, "chunk": self.chunk,
                "layout": self.layout, "rank": self.rank, "causal": self.causal,
                "alibi": self.alibi, "input_std": self.std, "backward": self.backward}


WORKLOADS = [
    Workload(1, "fp32-h1-d64-s256-n4-contiguous-r2", "fp32", 1, 1, 1, 64, 256, 4, "contiguous", 2),
    Workload(2, "bf16-h32-d128-s16k-n8-zigzag-r7", "bf16", 1, 32, 32, 128, 16384, 8, "zigzag", 7),
    Workload(3, "bf16-h32-d128-s128k-n8-zigzag-r7", "bf16", 1, 32, 32, 128, 131072, 8, "zigzag", 7),
    Workload(4, "bf16-gqa64x8-d128-s64k-n4-contiguous-r3-alibi", "bf16", 1, 64, 8, 128, 65536, 4,
             "contiguous", 3, alibi=True, std=math.sqrt(0.5)),
    Workload(5, "bf16-h16-d128-s1m-n64-zigzag-r63-fwdbwd", "bf16", 1, 16, 16, 128, 1048576, 64,
             "zigzag", 63, backward=True),
    # The GQA + ALiBi contiguous share with its backward step (the backward on
    # the contiguous / GQA / ALiBi configuration).
    Workload(6, "bf16-gqa64x8-d128-s64k-n4-contiguous-r3-alibi-fwdbwd", "bf16", 1, 64, 8, 128, 65536, 4,
             "contiguous", 3, alibi=True, std=math.sqrt(0.5), backward=True),
]

BY_NAME = {w.name: w for w in WORKLOADS}
HEADLINE = WORKLOADS[2]


def get(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS[key - 1]
    return BY_NAME[key]
