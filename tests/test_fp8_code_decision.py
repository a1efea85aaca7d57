"""The e4m3 code decision of the quantiser kernel, checked exhaustively on the
CPU (no GPU needed).

The kernel does not divide per element: it forms x * fl(448 / amax) in fp32
(with x and amax first scaled by 2^64 when amax < 2^-64), rounds that to 16
significant bits by adding 0x80 to the bit pattern and clearing the low 8
bits, and converts the result to e4m3 with round-to-nearest-even. The claim
is that this equals RNE(448 x / amax) of the exact quotient, the code the
oracle defines, for every pair of bf16 values with |x| <= amax. Here that
fp32 arithmetic is replayed with numpy float32 (IEEE round-to-nearest-even,
subnormals kept, as the kernel is built) for every bf16 significand of amax
at several binades, against every bf16 x within 24 binades below amax (and
the exact zero), and compared with the oracle's code of the exact quotient.
Dropping the snap, snapping to 11 or fewer significant bits, or dropping the
pre-scale for tiny blocks each fails here."""
import numpy as np
import pytest

from oracle import e4m3_round

F32 = np.float32


def _bf16_values(exponents) -> np.ndarray:
    """All positive bf16 values (8-bit significands) with these binade
    exponents, as float32; exponent -127 means the bf16 subnormals."""
    out = []
    for e in exponents:
        if e == -127:
            m = np.arange(1, 128, dtype=np.uint32)          # subnormal fraction bits
            out.append((m << 16).view(np.float32))
        else:
            frac = np.arange(128, dtype=np.uint32)
            bits = (np.uint32(e + 127) << 23) | (frac << 16)
            out.append(bits.view(np.float32))
    return np.concatenate(out)


def _kernel_codes(x: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """The kernel's float32 steps, then RNE to e4m3 of the snapped value."""
    x = x.astype(F32)
    amax = amax.astype(F32)
    pre = np.where(amax < F32(2.0 ** -64), F32(2.0 ** 64), F32(1.0)).astype(F32)
    with np.errstate(divide="ignore"):
        mul = np.where(amax > 0, F32(448.0) / (amax * pre), F32(0.0)).astype(F32)
    y = ((x * pre).astype(F32) * mul).astype(F32)
    bits = y.view(np.uint32)
    snapped = ((bits + np.uint32(0x80)) & np.uint32(0xFFFFFF00)).view(np.float32)
    return e4m3_round(snapped.astype(np.float64))


def _exact_codes(x: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """The oracle's definition: RNE(448 x / amax), 448 x and amax exact in
    float64 and the quotient decided by one correctly rounded division."""
    return e4m3_round(448.0 * x.astype(np.float64) / amax.astype(np.float64))


@pytest.mark.parametrize("amax_exp", [-127, -126, -100, -65, -64, -20, 0, 8, 100, 127])
def test_reciprocal_snap_matches_exact_rne(amax_exp):
    amaxes = _bf16_values([amax_exp])
    lo = max(-127, amax_exp - 24)
    xs = _bf16_values(range(lo, amax_exp + 1) if lo > -127 else [-127] + list(range(-126, amax_exp + 1)))
    xs = np.concatenate([[F32(0.0)], xs, -xs])
    checked = 0
    for a in amaxes:
        sel = xs[np.abs(xs) <= a]
        amax = np.full(sel.shape, a, dtype=F32)
        got, want = _kernel_codes(sel, amax), _exact_codes(sel, amax)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (float(a), float(sel[bad[0]]), got[bad[0]], want[bad[0]])
        checked += sel.size
    assert checked >= 3 * amaxes.size            # at least 0, a and -a for every amax


@pytest.mark.parametrize("amax", [448.0, 24.5, 24.5 * 2.0 ** -70])
def test_ties_go_to_even(amax):
    """x = m amax / 448 puts the quotient exactly on each e4m3 midpoint m; with
    amax = 24.5 (or 24.5 * 2^-70, the pre-scaled path) 448 / amax is not exact
    in fp32, x = 7 m / 128 still fits bf16's 8 significant bits, and 30 of the
    126 ties land off the midpoint when the product is not snapped. Every tie
    must go to the neighbour with the even significand."""
    vals = [m * 2.0 ** -9 for m in range(8)]                         # 0 and the subnormals
    vals += [(1 + m / 8) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
    grid = np.array([v for v in vals if v <= 448.0])
    mids = (grid[:-1] + grid[1:]) / 2
    x = (mids * amax / 448.0).astype(F32)
    assert np.array_equal(x.astype(np.float64), mids * amax / 448.0)      # exact
    assert np.all((x.view(np.uint32) & np.uint32(0xFFFF)) == 0)           # bf16 values
    amaxes = np.full(x.shape, amax, dtype=F32)
    got = _kernel_codes(x, amaxes)
    assert np.array_equal(got, _exact_codes(x, amaxes))
    lower, upper = grid[:-1], grid[1:]
    assert np.all((got == lower) | (got == upper))
    ulp = np.power(2.0, np.floor(np.log2(np.maximum(got, 2.0 ** -6))) - 3)
    assert np.all(np.mod(got / ulp, 2) == 0)
    assert np.any(got == lower) and np.any(got == upper)
