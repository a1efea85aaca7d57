"""Decoded frames to contiguous uint8: FP32 BCTHW -> uint8 BTHWC.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline leg may import or call this module; the product path never does.

Source: "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长", section
"紧凑输出与并行 MP4 构建", and "MiniMax H3 FastH3 real-time serving with
vLLM-Omni", section "System-wide optimizations in vLLM-Omni" (GPU output
preparation bullet): the decoder's FP32 BCTHW frames are converted once, on
the GPU, to uint8 BTHWC (a quarter of the bytes) before they go to the host.

The pages give neither the value range nor the rounding. Reading taken (the
usual convention for decoded video in [-1, 1]):
    u = round_half_even(255 * clamp(x / 2 + 1/2, 0, 1)),
the exact value of this expression for the float32 input x (no intermediate
rounding), NaN mapping to 0. Layout: x[b, c, t, h, w] -> u[b, t, h, w, c].

For x in (-1, 1) the level is RNE(255 (1 + x) / 2). Writing x = M 2^E with M
an integer of at most 24 bits, 255 (1 + x) / 2 = 255 (2^-E + M) / 2^(1-E),
an integer over a power of two, so the rounding is decided exactly on
integers: quotient, remainder, and the remainder compared with half the
divisor (equal: a tie, which goes to the even quotient). This is done for
|x| >= 2^-16 (2^-E <= 2^40, so everything fits in int64); for smaller |x| the
value lies within 0.002 of 127.5, below it exactly when x < 0, so the level
is 127 for negative x and 128 otherwise (x = 0 gives 127.5 exactly, a tie,
and goes to the even 128).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def frames_to_uint8_values(x) -> np.ndarray:
    """The exact per-element map (any shape), as uint8."""
    x = np.asarray(x, dtype=F32)
    xd = x.astype(np.float64)                       # exact
    out = np.zeros(x.shape, dtype=np.uint8)         # x <= -1, -inf and NaN give 0
    out[xd >= 1.0] = 255
    inner = (xd > -1.0) & (xd < 1.0)
    v = xd[inner]
    m, e = np.frexp(v)                              # v = m 2^e, 0.5 <= |m| < 1 (or 0)
    big_m = np.rint(np.ldexp(m, 24)).astype(np.int64)   # exact integer, |M| < 2^24
    shift = 24 - e.astype(np.int64)                 # v = M 2^-shift
    u = np.where(v < 0, 127, 128).astype(np.int64)  # |v| < 2^-16
    ok = shift <= 40
    s = shift[ok]
    num = 255 * ((np.int64(1) << s) + big_m[ok])    # 255 (1 + v) 2^s, an exact integer
    q = num >> (s + 1)                              # floor(255 (1 + v) / 2)
    r = num & ((np.int64(1) << (s + 1)) - 1)
    half = np.int64(1) << s
    u[ok] = q + (r > half) + ((r == half) & ((q & 1) == 1))
    out[inner] = u.astype(np.uint8)
    return out


def frames_to_uint8_bthwc(x) -> np.ndarray:
    """x float32 [B, C, T, H, W] -> uint8 [B, T, H, W, C]."""
    x = np.asarray(x, dtype=F32)
    if x.ndim != 5:
        raise ValueError("x must be [B, C, T, H, W]")
    return np.ascontiguousarray(frames_to_uint8_values(x).transpose(0, 2, 3, 4, 1))
