"""Pins of the MXFP4 emulation (OCP MX v1.0 reading: 32-element blocks along
K, E8M0 shared scale 2^(floor(log2 amax) - 2), E2M1 elements, round to
nearest even, saturating at +-6), CPU only."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import (E2M1_VALUES, e2m1_round, mx_dequantize, mxfp4_codes, mxfp4_fake_quant,
                    mxfp4_linear_ref, mxfp4_quantize, mxfp4_scale_exponents)


def _nearest_even_code(v: float) -> float:
    """Independent rounding: the E2M1 magnitude nearest to |v| by exact
    rational distance, a tie going to the even index, |v| > 6 to 6."""
    a = abs(Fraction(v))
    best = None
    for i, g in enumerate(E2M1_VALUES):
        d = abs(a - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    mag = E2M1_VALUES[best[1]]
    return -mag if v < 0 else mag


@pytest.mark.parametrize("v,want", [
    (0.0, 0.0), (0.25, 0.0), (0.2500001, 0.5), (0.5, 0.5), (0.75, 1.0), (0.7499, 0.5),
    (1.25, 1.0), (1.2501, 1.5), (1.75, 2.0), (2.5, 2.0), (2.51, 3.0), (3.5, 4.0), (3.49, 3.0),
    (5.0, 4.0), (5.01, 6.0), (6.0, 6.0), (7.99, 6.0), (100.0, 6.0), (-0.1, -0.0), (-1.75, -2.0),
    (-5.0, -4.0), (-7.0, -6.0)])
def test_e2m1_rounding_table(v, want):
    """Hand-worked: the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 go to
    the value with the even index (0, 1, 1, 2, 2, 4, 4); above 5 every
    value saturates to 6."""
    got = float(e2m1_round(v))
    assert got == want and np.signbit(got) == np.signbit(want)


def test_e2m1_grid_points_are_fixed_points_and_brute_force():
    g = np.array(E2M1_VALUES)
    assert np.array_equal(e2m1_round(g), g) and np.array_equal(e2m1_round(-g), -g)
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-8, 8, 3000), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 
                        rng.choice([-1.0, 1.0], 7)])
    got = e2m1_round(v)
    want = np.array([_nearest_even_code(float(x)) for x in v])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("amax,exp", [(6.0, 0), (4.0, 0), (7.99, 0), (8.0, 1), (3.99, -1), (1.0, -2),
                                      (0.75, -3), (2.0 ** 100, 98), (2.0 ** -124, -126),
                                      (2.0 ** -130, -127)])
def test_scale_exponent_rule(amax, exp):
    """floor(log2 amax) - 2, raised to -127 where lower."""
    x = np.zeros((1, 32))
    x[0, 9] = -amax
    x[0, 2] = amax / 5
    assert int(mxfp4_scale_exponents(x)[0, 0]) == exp


def test_zero_block_and_codes():
    """All-zero block: exponent -127, codes 0 (8 for negative zero);
    signs come from the input, also where the value rounds to zero."""
    x = np.zeros((1, 64))
    x[0, 33] = 6.0
    x[0, 34] = -0.1          # rounds to -0 at scale 1
    x[0, 35] = -3.0
    x[0, 36] = 2.5           # tie -> 2 (index 4)
    x[0, 1] = -0.0
    codes, e = mxfp4_codes(x)
    assert e.tolist() == [[-127, 0]]
    assert codes[0, 0] == 0 and codes[0, 1] == 8
    assert codes[0, 33] == 7 and codes[0, 34] == 8 and codes[0, 35] == 8 + 5 and codes[0, 36] == 4


def test_round_trip_of_representable_blocks():
    """V = 2^s P with P on the E2M1 grid and max |P| in {4, 6}: the block's
    exponent is s and the elements come back unchanged."""
    rng = np.random.default_rng(13)
    grid = np.concatenate([-np.array(E2M1_VALUES)[::-1], np.array(E2M1_VALUES)[1:]])
    for _ in range(50):
        s = int(rng.integers(-100, 100))
        p = rng.choice(grid, size=32)
        p[rng.integers(32)] = rng.choice([4.0, -4.0, 6.0, -6.0])
        v = p * 2.0 ** s
        pq, e = mxfp4_quantize(v[None, :])
        assert int(e[0, 0]) == s
        assert np.array_equal(pq[0], p)
        assert np.array_equal(mx_dequantize(pq, e)[0], v)


def test_saturation_and_error_bound():
    """Elements of a block are within half a spacing of V / X (spacing 0.5
    below 2, 1 in [2, 4), 2 in [4, 6]) or saturated at 6 X, and a block
    does not see its neighbours."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((8, 256)) * np.power(10.0, rng.uniform(-3, 3, (8, 1)))
    p, e = mxfp4_quantize(x)
    scale = np.repeat(np.power(2.0, e.astype(float)), 32, axis=-1)
    v = x / scale
    assert np.all(np.abs(v) < 8)
    sp = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    err = np.abs(p - v)
    assert np.all((err <= sp / 2 + 1e-12) | (np.abs(p) == 6.0))
    y = x.copy()
    y[:, 32:64] *= 1000.0
    p2, _ = mxfp4_quantize(y)
    assert np.array_equal(p2[:, :32], p[:, :32]) and np.array_equal(p2[:, 64:], p[:, 64:])


def test_mxfp4_linear_blockwise_brute_force():
    """y = sum over blocks of X_a X_w (P_a . P_w), with loops over rows,
    columns and blocks."""
    rng = np.random.default_rng(19)
    a = rng.standard_normal((5, 96)) * 3
    w = rng.standard_normal((4, 96)) * 0.02
    pa, ea = mxfp4_quantize(a)
    pw, ew = mxfp4_quantize(w)
    want = np.zeros((5, 4))
    for i in range(5):
        for j in range(4):
            for b in range(3):
                sl = slice(32 * b, 32 * b + 32)
                want[i, j] += 2.0 ** (ea[i, b] + ew[j, b]) * float(pa[i, sl] @ pw[j, sl])
    assert np.allclose(mxfp4_linear_ref(a, w), want, rtol=0, atol=1e-12)
    assert np.array_equal(mxfp4_fake_quant(a), mx_dequantize(pa, ea))


def test_mxfp4_error_level_against_exact_linear():
    """E2M1 keeps one mantissa bit: on i.i.d. operands the MXFP4 product is
    roughly 10-20 % (relative Frobenius error) from the exact one, several
    times the MXFP8 error."""
    rng = np.random.default_rng(23)
    a = rng.standard_normal((64, 512))
    w = rng.standard_normal((48, 512)) * 0.02
    exact = a @ w.T
    err = np.linalg.norm(mxfp4_linear_ref(a, w) - exact) / np.linalg.norm(exact)
    assert 0.05 < err < 0.3
