"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and nothing else. It holds none of the
attention arithmetic (no positions, layouts, masks, scales or slopes), which
is why both the fp64 oracle side and the GPU side may take their inputs from
it while sharing no other code.

Recipe: every tensor is drawn in float32 from N(0, std^2) by a
``torch.Generator`` seeded with the tensor's own seed, on the device it is
asked for, and then rounded to the working dtype (round-to-nearest-even for
bfloat16). The oracle consumes host copies of exactly these rounded values,
upcast to float64. CPU and CUDA generators give different streams for the
same seed; a test or benchmark draws each tensor once and hands the same
values to both sides.

Seeds: tensor ``i`` of workload ``k`` uses ``1000 * k + i`` with i = 0, 1, 2, 3
for Q, K, V and the output gradient dO.
"""

from __future__ import annotations

import torch

Q_STREAM, K_STREAM, V_STREAM, DO_STREAM = 0, 1, 2, 3

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    try:
        return _DTYPES[name]
    except KeyError:
        raise ValueError(f"unknown dtype {name!r}") from None


def seed_for(workload_index: int, stream: int) -> int:
    return 1000 * int(workload_index) + int(stream)


def normal(shape, seed: int, std: float = 1.0, dtype: str = "fp32", device="cpu") -> torch.Tensor:
    """float32 draws from N(0, std^2), rounded to ``dtype`` (RNE)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(float(std))
    return x.to(torch_dtype(dtype))
