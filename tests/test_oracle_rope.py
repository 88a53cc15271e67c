"""Pins for the RoPE oracle, each independent of the oracle's own formula:

* the same rotation written as complex multiplication (numpy complex128),
* the same rotation as a block 2x2 rotation matrix applied with a matmul,
* position 0 is the identity, and rotation preserves each pair's norm,
* the rotation group law: rotating by a then by b equals rotating by a + b,
* the relative-position property the page states: <R_m q, R_n k> depends on
  m - n only,
* a planted mistake (sine sign flipped, or the halves paired as neighbours)
  fails the complex-number pin.
"""

import numpy as np
import pytest

import oracle
from oracle import rope_fp64


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_matches_complex_multiplication(d):
    x = _rand((3, 17, d), 1)
    pos = np.array([0, 1, 2, 5, 63, 64, 100, 1000, 4095, 4096, 65535, 131071, 200000, 524287, 1048575,
                    1048576, 999999])
    got = oracle.rotary_embedding(x, pos)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    theta = 10000.0 ** (-(2.0 * np.arange(d // 2)) / d)
    w = z * np.exp(1j * np.outer(pos, theta))
    ref = np.concatenate([w.real, w.imag], axis=-1)
    assert np.max(np.abs(got - ref)) < 1e-9


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


@pytest.mark.parametrize("mistake", ["sine_sign", "neighbour_pairs"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    def flawed(x, positions, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_fp64.inv_freq(d, base)[None, :]
        cos, sin = np.cos(ang), np.sin(ang)
        if mistake == "sine_sign":
            x1, x2 = x[..., : d // 2], x[..., d // 2:]
            return np.concatenate([x1 * cos + x2 * sin, -x1 * sin + x2 * cos], axis=-1)
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2], out[..., 1::2] = x1 * cos - x2 * sin, x1 * sin + x2 * cos
        return out

    monkeypatch.setattr(oracle, "rotary_embedding", flawed)
    with pytest.raises(AssertionError):
        test_matches_complex_multiplication(8)
