"""Shared helpers of the parity tests: draw seeded inputs, run the HIP path
through the C ABI, run the fp64 oracle on host copies of the same values."""

from __future__ import annotations

import json
import math
import os
import sys
import time
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import seeded_inputs as si


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    dtype: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_len: int
    n_ranks: int
    layout: str
    causal: bool = True
    alibi: bool = False
    std: float = 1.0
    seed: int = 0
    scale: float = None
    extra: dict = field(default_factory=dict)

    @property
    def chunk(self):
        return self.seq_len // self.n_ranks

    def sc(self):
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def tag(self):
        return (f"{self.dtype} B{self.batch} H{self.heads_q}/{self.heads_kv} D{self.head_dim} S{self.seq_len} "
                f"N{self.n_ranks} {self.layout} causal={self.causal} alibi={self.alibi} seed={self.seed}")


def draw(case: Case, device="cuda", with_do=False):
    """Global-order inputs on `device` (seeded), plus dO for the rank chunk."""
    shp_q = (case.batch, case.heads_q, case.seq_len, case.head_dim)
    shp_k = (case.batch, case.heads_kv, case.seq_len, case.head_dim)
    q = si.normal(shp_q, si.seed_for(case.seed, si.Q_STREAM), case.std, case.dtype, device)
    k = si.normal(shp_k, si.seed_for(case.seed, si.K_STREAM), case.std, case.dtype, device)
    v = si.normal(shp_k, si.seed_for(case.seed, si.V_STREAM), case.std, case.dtype, device)
    if not with_do:
        return q, k, v
    shp_do = (case.batch, case.heads_q, case.chunk, case.head_dim)
    do = si.normal(shp_do, si.seed_for(case.seed, si.DO_STREAM), 1.0, case.dtype, device)
    return q, k, v, do


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def host_heads(t: torch.Tensor, heads) -> np.ndarray:
    """float32 host copy holding only the listed heads (others left as zeros
    that are never touched, so they cost no physical memory)."""
    out = np.zeros(tuple(t.shape), dtype=np.float32)
    for h in sorted(set(int(x) for x in heads)):
        out[:, h] = t[:, h].to("cpu", torch.float32).numpy()
    return out


def oracle_slopes(case: Case):
    return oracle.alibi_slopes(case.heads_q) if case.alibi else None


def max_abs(a, b) -> float:
    """Largest |a - b|; equal infinities count as 0, any NaN as +inf."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {b.shape}")
    if a.size == 0:
        return 0.0
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    d = np.where(np.isnan(d), np.inf, d)
    return float(d.max())


def record(config: str, rank: int, errors: dict, **extra) -> None:
    """Append one JSON line (config, rank, error figures, seeds, versions) to
    the file named by RA_PARITY_RECORD, when that is set."""
    path = os.environ.get("RA_PARITY_RECORD")
    if not path:
        return
    rec = {"config": config, "rank": int(rank), **{k: float(v) for k, v in errors.items()},
           "torch": torch.__version__, "hip": getattr(torch.version, "hip", None), **extra}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *exc):
        log(f"  {self.what}: {time.time() - self.t:.2f}s")
