"""CPU replay of the frame-compaction kernel's level decision (frames.hip):
y = 127.5 + 127.5 x with the product exact and one rounding of the sum in
float64 (the fma), clamped to [0, 255] and rounded to nearest even; for
|x| < 2^-20 the sign of x decides between 127 and 128. The replay must equal
the oracle's exact map on a strided sweep of fp32 bit patterns in (-2, 2),
on the values next to every midpoint and on tiny values of both signs."""
import numpy as np

from oracle import frames_to_uint8_values

F32 = np.float32


def _kernel_steps(x: np.ndarray) -> np.ndarray:
    y = 127.5 * x.astype(np.float64) + 127.5
    y = np.minimum(np.maximum(np.nan_to_num(y, nan=0.0), 0.0), 255.0)
    u = np.rint(y).astype(np.int64)
    u = np.where(np.abs(x) < F32(2.0 ** -20), np.where(x < 0, 127, 128), u)
    u = np.where(x >= 1, 255, u)
    return np.where(x > -1, u, 0).astype(np.uint8)


def test_strided_sweep_of_all_fp32_inputs():
    for sign in (0, 1):
        bits = np.arange(0, 0x40000000, 61, dtype=np.uint32) | np.uint32(sign << 31)
        x = bits.view(F32)
        assert np.array_equal(_kernel_steps(x), frames_to_uint8_values(x))


def test_next_to_midpoints_and_tiny():
    vals = []
    for k in range(255):
        c = np.float32((2 * k + 1) / 255.0 - 1.0)
        lo = hi = c
        vals.append(c)
        for _ in range(64):
            lo = np.nextafter(lo, F32(-2), dtype=F32)
            hi = np.nextafter(hi, F32(2), dtype=F32)
            vals += [lo, hi]
    vals += [s * 2.0 ** -n for n in range(1, 150) for s in (1.0, -1.0)] + [0.0, -0.0, np.nan,
                                                                           np.inf, -np.inf]
    x = np.array(vals, F32)
    assert np.array_equal(_kernel_steps(x), frames_to_uint8_values(x))
