"""Pins of the frame compaction oracle (FP32 BCTHW -> uint8 BTHWC), CPU only.

The map is u = round_half_even(255 * clamp(x / 2 + 1/2, 0, 1)), NaN -> 0,
taken exactly for the float32 input; the pins compare it with Python's
exact rational arithmetic (fractions.Fraction, whose round() goes to the
even integer on ties)."""
from fractions import Fraction

import numpy as np

from oracle import frames_to_uint8_bthwc, frames_to_uint8_values


def _exact_level(x: float) -> int:
    """The definition in exact rational arithmetic, one value at a time."""
    if x != x:
        return 0
    if x in (float("inf"), float("-inf")):
        return 255 if x > 0 else 0
    y = Fraction(x) / 2 + Fraction(1, 2)
    y = min(max(y, Fraction(0)), Fraction(1))
    return round(255 * y)


def _near_midpoints() -> np.ndarray:
    """float32 inputs next to every midpoint: the nearest float32 to
    (2k + 1) / 255 - 1 (255 (1 + x) / 2 = k + 1/2) and its 4 neighbours on
    each side."""
    out = []
    for k in range(255):
        c = np.float32((2 * k + 1) / 255.0 - 1.0)
        for step in range(-4, 5):
            v = c
            for _ in range(abs(step)):
                v = np.nextafter(v, np.float32(np.inf if step > 0 else -np.inf), dtype=np.float32)
            out.append(v)
    return np.array(out, np.float32)


def _tiny() -> np.ndarray:
    mags = [2.0 ** -n for n in range(14, 150)] + [1e-45, 3e-45, 1.17e-38]
    return np.array([s * m for m in mags for s in (1.0, -1.0)] + [0.0, -0.0], np.float32)


def test_fixed_points_and_clamp():
    x = np.array([-1.0, 1.0, 0.0, -7.5, 3.0, np.inf, -np.inf, np.nan, -0.0], np.float32)
    # 0 -> 127.5 exactly, a tie, which goes to the even 128
    assert frames_to_uint8_values(x).tolist() == [0, 255, 128, 0, 255, 255, 0, 0, 128]


def test_exact_against_rational_arithmetic():
    """Random values, values next to every midpoint (either side, and the
    float32 nearest to it), tiny values of both signs down to the smallest
    subnormal, signed zeros and the ends: every level equals the exact
    rational definition."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-1.2, 1.2, 20000).astype(np.float32), _near_midpoints(), _tiny(),
                        np.array([-1.0, 1.0, np.nextafter(np.float32(-1), np.float32(0)),
                                  np.nextafter(np.float32(1), np.float32(0)), np.nan, np.inf, -np.inf],
                                 np.float32)])
    got = frames_to_uint8_values(x)
    want = np.array([_exact_level(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, want)


def test_tiny_negative_values_round_down():
    """255 (1 + x) / 2 is just below the midpoint 127.5 for every negative
    x, so the level is 127 however small |x| is; a float32 evaluation of
    x * 0.5 + 0.5 would return 128 below |x| = 2^-25."""
    x = np.array([-2.0 ** -30, -1e-45, -2.0 ** -17], np.float32)
    assert frames_to_uint8_values(x).tolist() == [127, 127, 127]
    assert frames_to_uint8_values(-x).tolist() == [128, 128, 128]


def test_every_level_is_reached_once_in_order():
    """The inverse images of the 256 levels partition [-1, 1] in order: a
    fine monotone sweep hits every level, never decreasing."""
    x = np.linspace(-1, 1, 200001, dtype=np.float32)
    u = frames_to_uint8_values(x).astype(int)
    assert np.all(np.diff(u) >= 0) and np.array_equal(np.unique(u), np.arange(256))


def test_layout_by_index_loops():
    rng = np.random.default_rng(8)
    x = rng.uniform(-1, 1, (2, 3, 2, 3, 5)).astype(np.float32)
    u = frames_to_uint8_bthwc(x)
    assert u.shape == (2, 2, 3, 5, 3) and u.dtype == np.uint8
    for b in range(2):
        for c in range(3):
            for t in range(2):
                for h in range(3):
                    for w in range(5):
                        assert u[b, t, h, w, c] == frames_to_uint8_values(x[b, c, t, h, w])
