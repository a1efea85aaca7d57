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
evaluated in IEEE float32 in exactly this order (x * 0.5, + 0.5, clamp,
* 255, round to nearest even), the precision the kernel uses, so that both
sides take the integer decision in the same arithmetic; NaN maps to 0
(IEEE max/min return the non-NaN operand). Layout: x[b, c, t, h, w] ->
u[b, t, h, w, c].
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def frames_to_uint8_values(x) -> np.ndarray:
    """The per-element map in float32 (any shape), as uint8."""
    x = np.asarray(x, dtype=F32)
    y = (x * F32(0.5)).astype(F32)
    y = (y + F32(0.5)).astype(F32)
    y = np.where(np.isnan(y), F32(0.0), y)
    y = np.minimum(np.maximum(y, F32(0.0)), F32(1.0)).astype(F32)
    z = (y * F32(255.0)).astype(F32)
    return np.rint(z).astype(np.uint8)      # rint: round half to even


def frames_to_uint8_bthwc(x) -> np.ndarray:
    """x float32 [B, C, T, H, W] -> uint8 [B, T, H, W, C]."""
    x = np.asarray(x, dtype=F32)
    if x.ndim != 5:
        raise ValueError("x must be [B, C, T, H, W]")
    return np.ascontiguousarray(frames_to_uint8_values(x).transpose(0, 2, 3, 4, 1))
