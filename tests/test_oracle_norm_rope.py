"""Pins of the oracle's RMSNorm, 3D RoPE and fused Q/K norm + RoPE (CPU)."""
import cmath
import math

import numpy as np
import pytest

from oracle import qk_norm_rope_ref, rmsnorm, rope_3d


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rmsnorm_known_value_and_rms():
    z = np.array([3.0, 4.0])
    assert np.allclose(rmsnorm(z, 0.0), z / math.sqrt(12.5), rtol=0, atol=1e-15)
    eps = 1e-6
    x = _rand((50, 96), 1)
    y = rmsnorm(x, eps)
    ms = np.mean(x * x, axis=1)
    rms = np.sqrt(np.mean(y * y, axis=1))
    assert np.max(np.abs(rms - np.sqrt(ms / (ms + eps)))) < 1e-14


def test_rmsnorm_scale_invariance_without_eps():
    x = _rand((10, 64), 2)
    assert np.max(np.abs(rmsnorm(7.5 * x, 0.0) - rmsnorm(x, 0.0))) < 1e-14


def test_rope_preserves_norm_and_identity_at_origin():
    split = (32, 48, 48)
    x = _rand((300, 4, 128), 3)
    pos = np.random.default_rng(4).integers(0, 2000, size=(300, 1, 3))
    y = rope_3d(x, pos, split, 1e4)
    assert np.max(np.abs(np.linalg.norm(y, axis=-1) - np.linalg.norm(x, axis=-1))) < 1e-12
    assert np.array_equal(rope_3d(x, np.zeros((300, 1, 3), int), split, 1e4), x)


def test_rope_relative_position_property():
    split = (16, 24, 24)
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for _ in range(20):
        p = rng.integers(0, 500, size=3)
        p2 = rng.integers(0, 500, size=3)
        lhs = np.dot(rope_3d(q, p, split, 1e4), rope_3d(k, p2, split, 1e4))
        rhs = np.dot(rope_3d(q, p - p2, split, 1e4), k)
        assert abs(lhs - rhs) < 1e-10


def test_rope_pair_is_complex_rotation_with_known_angles():
    # split (4, 2, 6): t-axis pair 1 turns at theta^(-2/4) = 0.01 rad per step
    # when theta = 1e4, so position 100 turns it by exactly 1 rad.
    split = (4, 2, 6)
    x = _rand((12,), 6)
    y = rope_3d(x, np.array([100, 0, 0]), split, 1e4)
    z = complex(x[2], x[3]) * cmath.exp(1j * 1.0)
    assert abs(complex(y[2], y[3]) - z) < 1e-12
    # t-axis pair 0 turns at 1 rad per step
    z0 = complex(x[0], x[1]) * cmath.exp(1j * 100.0)
    assert abs(complex(y[0], y[1]) - z0) < 1e-11
    # everything outside the t slice is untouched at h = w = 0
    assert np.array_equal(y[4:], x[4:])
    # h axis: only dims [4, 6) move; w axis pair 2 of 3 has rate theta^(-4/6)
    y = rope_3d(x, np.array([0, 3, 0]), split, 1e4)
    assert np.array_equal(y[:4], x[:4]) and np.array_equal(y[6:], x[6:])
    assert abs(complex(y[4], y[5]) - complex(x[4], x[5]) * cmath.exp(3j)) < 1e-12
    y = rope_3d(x, np.array([0, 0, 1000]), split, 1e4)
    rate = 1e4 ** (-4.0 / 6.0)          # = 10^(-8/3)
    assert abs(complex(y[10], y[11]) - complex(x[10], x[11]) * cmath.exp(1j * 1000 * rate)) < 1e-12


def test_rope_pairs_are_interleaved():
    # a quarter turn maps e_2 to e_3 (its interleaved partner), not to e_{2+D/2}
    split = (4, 0, 0)
    x = np.zeros(4)
    x[2] = 1.0
    pos = np.array([50.0 * math.pi, 0, 0])   # 0.01 rad/step * 50 pi = pi/2
    y = rope_3d(x, pos, split, 1e4)
    assert np.allclose(y, [0, 0, 0, 1], atol=1e-12)


def test_rope_rejects_bad_split():
    with pytest.raises(ValueError):
        rope_3d(np.zeros(64), np.zeros(3), (16, 24, 25), 1e4)
    with pytest.raises(ValueError):
        rope_3d(np.zeros(64), np.zeros(3), (15, 25, 24), 1e4)


def test_qk_norm_is_per_head_with_shared_gains():
    n, heads, d = 3, 2, 64
    q = np.ones((n, heads, d))
    q[:, 0, :] *= 10.0
    k = _rand((n, heads, d), 7)
    w = np.ones(d)
    w[0] = 2.0
    zero = np.zeros((n, 3), int)
    qo, ko = qk_norm_rope_ref(q, k, w, np.ones(d), zero, (16, 24, 24), 1e4, 0.0)
    # both heads normalise to unit rms on their own, then share the gain
    expect = np.ones(d)
    expect[0] = 2.0
    assert np.allclose(qo, expect[None, None, :], atol=1e-14)
    assert np.allclose(np.mean(ko * ko, axis=-1), 1.0, atol=1e-13)


def test_qk_norm_then_rope_order():
    # RoPE after the norm: the norm of the result equals the norm of the gained
    # RMS-normalised vector, and the position moves only q/k, per token
    n, heads, d = 5, 3, 64
    q, k = _rand((n, heads, d), 8), _rand((n, heads, d), 9)
    wq, wk = 1 + 0.1 * _rand(d, 10), 1 + 0.1 * _rand(d, 11)
    grid = np.random.default_rng(12).integers(0, 100, size=(n, 3))
    eps = 1e-6
    qo, ko = qk_norm_rope_ref(q, k, wq, wk, grid, (16, 24, 24), 1e4, eps)
    qn = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps) * wq
    assert np.allclose(np.linalg.norm(qo, axis=-1), np.linalg.norm(qn, axis=-1), atol=1e-12)
    q0, _ = qk_norm_rope_ref(q, k, wq, wk, np.zeros_like(grid), (16, 24, 24), 1e4, eps)
    assert np.allclose(q0, qn, atol=1e-13)
