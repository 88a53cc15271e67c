"""Pins for the RoPE oracle, each independent of the oracle's own formula
(which multiplies complex numbers):

* each pair turned element by element in pure Python with math.cos / math.sin,
* the same rotation as a block 2x2 rotation matrix applied with a matmul,
* position 0 is the identity, and rotation preserves each pair's norm,
* the rotation group law: rotating by a then by b equals rotating by a + b,
* the relative-position property the page states: <R_m q, R_n k> depends on
  m - n only,
* a planted mistake (sine sign flipped, the halves paired as neighbours, or
  the frequency exponent off by one pair) fails the element-by-element pin.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import rope_fp64


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


POSITIONS = [0, 1, 2, 5, 63, 64, 100, 1000, 4095, 4096, 65535, 131071, 200000, 524287, 1048575, 1048576, 999999]


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_matches_elementwise_rotation(d):
    x = _rand((2, len(POSITIONS), d), 1)
    got = oracle.rotary_embedding(x, np.array(POSITIONS))
    h = d // 2
    worst = 0.0
    for b in range(x.shape[0]):
        for t, p in enumerate(POSITIONS):
            for j in range(h):
                a = p * math.pow(10000.0, -2.0 * j / d)
                c, s_ = math.cos(a), math.sin(a)
                x1, x2 = float(x[b, t, j]), float(x[b, t, j + h])
                worst = max(worst, abs(got[b, t, j] - (x1 * c - x2 * s_)),
                            abs(got[b, t, j + h] - (x1 * s_ + x2 * c)))
    assert worst < 1e-9


def test_matches_rotation_matrices():
    d = 16
    x = _rand((5, d), 2)
    pos = np.array([3, 17, 256, 9999, 123456])
    got = oracle.rotary_embedding(x, pos, base=500.0)
    for r in range(5):
        R = np.zeros((d, d))
        for j in range(d // 2):
            a = pos[r] * 500.0 ** (-2.0 * j / d)
            R[np.ix_([j, j + d // 2], [j, j + d // 2])] = [[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]]
        assert np.max(np.abs(got[r] - R @ x[r])) < 1e-12


def test_identity_at_zero_and_norm_preserved():
    x = _rand((4, 9, 32), 3)
    assert np.array_equal(oracle.rotary_embedding(x, np.zeros(9, dtype=np.int64)), x)
    y = oracle.rotary_embedding(x, np.arange(9) * 7919)
    n_x = x[..., :16] ** 2 + x[..., 16:] ** 2
    n_y = y[..., :16] ** 2 + y[..., 16:] ** 2
    assert np.max(np.abs(n_x - n_y)) < 1e-12


def test_group_law():
    x = _rand((2, 6, 64), 4)
    a = np.array([0, 5, 77, 1024, 30000, 500000])
    b = np.array([9, 1, 3000, 2, 65536, 500000])
    two = oracle.rotary_embedding(oracle.rotary_embedding(x, a), b)
    one = oracle.rotary_embedding(x, a + b)
    assert np.max(np.abs(two - one)) < 1e-9


def test_relative_position_property():
    d = 128
    q, k = _rand((d,), 5), _rand((d,), 6)
    for m, n in [(10, 3), (1000, 993), (1048575, 1048568)]:
        dot = float(oracle.rotary_embedding(q[None], np.array([m]))[0] @ oracle.rotary_embedding(k[None], np.array([n]))[0])
        ref = float(oracle.rotary_embedding(q[None], np.array([m - n]))[0] @ k)
        assert abs(dot - ref) < 1e-9 * (1 + abs(ref))


@pytest.mark.parametrize("mistake", ["sine_sign", "neighbour_pairs", "exponent"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    true_rope = rope_fp64.rotary_embedding

    def flawed(x, positions, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        if mistake == "sine_sign":
            return true_rope(x, -np.asarray(positions), base)
        if mistake == "exponent":  # theta_j = base^(-2(j+1)/d): every plane one step too slow
            h = d // 2
            theta = base ** (-2.0 * (np.arange(h) + 1.0) / d)
            w = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.multiply.outer(np.asarray(positions, float), theta))
            return np.concatenate([w.real, w.imag], axis=-1)
        out = np.empty_like(x)
        nb = true_rope(np.concatenate([x[..., 0::2], x[..., 1::2]], axis=-1), positions, base)
        out[..., 0::2], out[..., 1::2] = nb[..., : d // 2], nb[..., d // 2:]
        return out

    monkeypatch.setattr(oracle, "rotary_embedding", flawed)
    with pytest.raises(AssertionError):
        test_matches_elementwise_rotation(8)
