"""Rotary position embedding in float64 (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; it imports nothing from the product package.

Follows the intelliparadigm.com long-context survey, §2.1.3 (RoPE的旋转位置编码):
the head dimension d is cut into a first and a second half, x1 = x[:d/2] and
x2 = x[d/2:]; element j of the first half pairs with element j of the second,
and the pair is turned by the angle p * theta_j, where p is the token position
and theta_j = base^(-2j/d) (base 10000 on that page):

    out[j]       = x1[j] cos(p theta_j) - x2[j] sin(p theta_j)
    out[j + d/2] = x1[j] sin(p theta_j) + x2[j] cos(p theta_j)

Reading: the page's listing forms the angles in float32, which at positions
near 10^6 is off by several hundredths of a radian; the oracle takes the exact
function (angles and trigonometry in float64). Positions are the tokens'
global positions, so a rank's rows under either layout carry the same
rotation as in the unsharded sequence.
"""

from __future__ import annotations

import numpy as np


def inv_freq(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_j = base^(-2j/d), j = 0 .. d/2 - 1 (survey §2.1.3, the inv_freq
    buffer of its RotaryEmbedding)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    return base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)


def rotary_embedding(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """RoPE of ``x`` ``[..., L, d]`` at the positions ``[L]`` (survey §2.1.3,
    apply_rotary_emb with the cos/sin of the RotaryEmbedding), in float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(d, base)[None, :]  # [L, d/2]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)
