"""Pins of the frame compaction oracle (FP32 BCTHW -> uint8 BTHWC), CPU only."""
import numpy as np

from oracle import frames_to_uint8_bthwc, frames_to_uint8_values


def test_fixed_points_and_clamp():
    x = np.array([-1.0, 1.0, 0.0, -7.5, 3.0, np.inf, -np.inf, np.nan, -0.0], np.float32)
    # 0 -> 127.5 exactly, a tie, which goes to the even 128
    assert frames_to_uint8_values(x).tolist() == [0, 255, 128, 0, 255, 255, 0, 0, 128]


def test_every_level_is_reached_once_in_order():
    """The inverse images of the 256 levels partition [-1, 1] in order: a
    fine monotone sweep hits every level, never decreasing."""
    x = np.linspace(-1, 1, 200001, dtype=np.float32)
    u = frames_to_uint8_values(x).astype(int)
    assert np.all(np.diff(u) >= 0) and np.array_equal(np.unique(u), np.arange(256))


def test_rounding_to_nearest_against_float64():
    """Away from the float32 rounding of a midpoint the level is the nearest
    integer to the exact 255 (x + 1) / 2."""
    x = np.random.default_rng(7).uniform(-1.2, 1.2, 100000).astype(np.float32)
    exact = 255.0 * np.clip(x.astype(np.float64) / 2 + 0.5, 0, 1)
    u = frames_to_uint8_values(x).astype(float)
    frac = np.abs(exact - np.floor(exact) - 0.5)
    clear = frac > 1e-4
    assert np.array_equal(u[clear], np.floor(exact[clear] + 0.5))
    assert np.all(np.abs(u - exact) <= 0.5 + 1e-4)


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
