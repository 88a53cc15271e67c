"""Rotary position embedding in float64 (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; it imports nothing from the product package.

Follows the intelliparadigm.com long-context survey, §2.1.3 (RoPE的旋转位置编码),
written here from the rotation it describes: the head dimension d is cut into
a first and a second half; element j of the first half and element j of the
second form one plane, read as the complex number z_j = x[j] + i x[j + d/2],
and that plane is turned by the angle p * theta_j, where p is the token
position and theta_j = base^(-2j/d) (base 10000 on that page). Turning a plane
by an angle a is multiplication by e^{ia}, so the output pair is the real and
imaginary part of z_j e^{i p theta_j}.

Reading: the page forms the angles in float32, which at positions near 10^6
is off by several hundredths of a radian; the oracle takes the exact function
(angles and the complex exponential in float64). Positions are the tokens'
global positions, so a rank's rows under either layout carry the same
rotation as in the unsharded sequence.
"""

from __future__ import annotations

import numpy as np


def inv_freq(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_j = base^(-2j/d), j = 0 .. d/2 - 1: the turning rate of plane j
    (survey §2.1.3)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / head_dim)


def rotary_embedding(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """RoPE of ``x`` ``[..., L, d]`` at the positions ``[L]`` (survey §2.1.3):
    each plane (j, j + d/2) of row t turned by positions[t] * theta_j, in
    float64 complex arithmetic."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    turn = np.exp(1j * np.multiply.outer(np.asarray(positions, dtype=np.float64), inv_freq(d, base)))  # [L, d/2]
    w = z * turn
    out = np.empty_like(x)
    out[..., :half] = w.real
    out[..., half:] = w.imag
    return out
