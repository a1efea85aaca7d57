"""Float64 emulation of MXFP8 (E4M3) linears for the DiT block GEMMs.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline leg may import or call this module; the product path never does.

Sources:
  [H3-950PR] "MiniMax H3 on Ascend 950PR / 950DT", section "Recommended lossy
      configuration": the transformer runs with MXFP8 online quantization.
  [FastH3-EN] "MiniMax H3 FastH3 real-time serving with vLLM-Omni", section
      "Scaling beyond the FastH3 profile", bullet "Quantization paths": online
      FP8 for the linear layers lowers peak HBM (~39 %) for a small latency gain.
  [FastH3-ZH] "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长", section
      "其他加速路径：有损但可控": some linear layers are quantised to FP8 at load
      time.

The pages name the method (MXFP8) but not its format. This module follows
the public OCP Microscaling Formats (MX) v1.0 specification, section on
converting a vector of values to an MX block:
  * blocks of 32 consecutive elements along the reduction (K) dimension;
  * shared scale X = 2^(floor(log2(max |V_i|)) - 8), 8 being the largest
    exponent of E4M3 (max normal 448 = 1.75 * 2^8), held as an E8M0 byte
    (exponent + 127); a block of zeros gets the smallest scale 2^-127, and an
    exponent below -127 is raised to -127;
  * elements P_i = E4M3(V_i / X): round to nearest even, saturating at
    +-448 (V_i / X can reach 511.9 when the block maximum is just under a
    power of two times 512);
  * the value of an element is X * P_i.
An MX linear y = a W^T multiplies the dequantised operands: both are
quantised along K, so every product pairs elements of the same block index
and y = sum over blocks of X_a X_w (P_a . P_w). Here that product is taken
in float64; the only freedom left to an implementation is the summation
order and precision.

MXFP4 ([H3-950PR] section "MXFP4 online quantization": the DiT's linears can
run with MXFP4 online quantization instead of MXFP8; again no format is
given) follows the same specification with E2M1 elements: blocks of 32
along K, shared scale X = 2^(floor(log2(max |V_i|)) - 2), 2 being the
largest exponent of E2M1 (max normal 6 = 1.5 * 2^2), the same E8M0 rules,
and elements P_i = E2M1(V_i / X) rounded to nearest even and saturating at
+-6 (V_i / X reaches 7.99). E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6,
index 0..7; a 4-bit code is (sign of V_i) * 8 + index, the sign taken from
V_i itself (a negative value that rounds to zero gives code 8).
"""
from __future__ import annotations

import numpy as np

from .fp8_attention import e4m3_round

_F = np.float64
MX_BLOCK = 32
E4M3_EMAX = 8
E2M1_EMAX = 2
E2M1_MAX = 6.0
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E8M0_BIAS = 127
E8M0_MIN_EXP = -127


def mx_scale_exponents(x, block: int = MX_BLOCK) -> np.ndarray:
    """Shared exponents floor(log2(amax)) - 8 of the blocks of the last axis
    (which must be a multiple of `block`), -127 for all-zero blocks and
    never below -127."""
    x = np.asarray(x, dtype=_F)
    k = x.shape[-1]
    if k % block:
        raise ValueError(f"last axis {k} is not a multiple of the block {block}")
    blocks = np.abs(x).reshape(*x.shape[:-1], k // block, block)
    amax = blocks.max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX
    e = np.where(amax > 0, e, E8M0_MIN_EXP)
    return np.maximum(e, E8M0_MIN_EXP).astype(np.int64)


def mx_quantize(x, block: int = MX_BLOCK):
    """(P, e): E4M3 element values P (float64, on the E4M3 grid) and the
    blocks' shared exponents e, so that the dequantised value of element j is
    P[..., j] * 2^e[..., j // block]."""
    x = np.asarray(x, dtype=_F)
    e = mx_scale_exponents(x, block)
    scale = np.repeat(np.power(2.0, e.astype(_F)), block, axis=-1)
    return e4m3_round(x / scale), e


def mx_dequantize(p, e, block: int = MX_BLOCK) -> np.ndarray:
    p = np.asarray(p, dtype=_F)
    return p * np.repeat(np.power(2.0, np.asarray(e, dtype=_F)), block, axis=-1)


def mx_fake_quant(x, block: int = MX_BLOCK) -> np.ndarray:
    """x rounded through MXFP8 and back (float64)."""
    p, e = mx_quantize(x, block)
    return mx_dequantize(p, e, block)


def mx_linear_ref(a, w, block: int = MX_BLOCK) -> np.ndarray:
    """y = dq(a) dq(w)^T with a [M, K] and w [N, K] each quantised along K."""
    return mx_fake_quant(a, block) @ mx_fake_quant(w, block).T


def e2m1_round(a) -> np.ndarray:
    """Round to the nearest E2M1 value (ties to the even code), saturating
    at +-6. Magnitudes in [2^e, 2^(e+1)) for e >= 0 are spaced 2^(e-1);
    below 1 the spacing stays 0.5 (the subnormal 0.5)."""
    a = np.asarray(a, dtype=_F)
    mag = np.abs(a)
    e = np.floor(np.log2(np.maximum(mag, 1.0)))
    ulp = np.power(2.0, e - 1)
    r = np.round(mag / ulp) * ulp            # numpy rounds halves to even
    r = np.minimum(r, E2M1_MAX)
    return np.copysign(r, a)


def mxfp4_scale_exponents(x, block: int = MX_BLOCK) -> np.ndarray:
    """Shared exponents floor(log2(amax)) - 2 of the blocks of the last axis,
    -127 for all-zero blocks and never below -127."""
    x = np.asarray(x, dtype=_F)
    k = x.shape[-1]
    if k % block:
        raise ValueError(f"last axis {k} is not a multiple of the block {block}")
    amax = np.abs(x).reshape(*x.shape[:-1], k // block, block).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E2M1_EMAX
    e = np.where(amax > 0, e, E8M0_MIN_EXP)
    return np.maximum(e, E8M0_MIN_EXP).astype(np.int64)


def mxfp4_quantize(x, block: int = MX_BLOCK):
    """(P, e): E2M1 element values P (float64) and the blocks' shared
    exponents e; element j dequantises to P[..., j] * 2^e[..., j // block]."""
    x = np.asarray(x, dtype=_F)
    e = mxfp4_scale_exponents(x, block)
    scale = np.repeat(np.power(2.0, e.astype(_F)), block, axis=-1)
    return e2m1_round(x / scale), e


def mxfp4_codes(x, block: int = MX_BLOCK):
    """(codes, e): the 4-bit element codes (uint8, sign * 8 + index of the
    magnitude in E2M1_VALUES, the sign being that of x) and the exponents."""
    x = np.asarray(x, dtype=_F)
    p, e = mxfp4_quantize(x, block)
    index = np.searchsorted(np.array(E2M1_VALUES), np.abs(p))
    return (np.signbit(x).astype(np.uint8) << 3) | index.astype(np.uint8), e


def mxfp4_fake_quant(x, block: int = MX_BLOCK) -> np.ndarray:
    """x rounded through MXFP4 and back (float64)."""
    p, e = mxfp4_quantize(x, block)
    return mx_dequantize(p, e, block)


def mxfp4_linear_ref(a, w, block: int = MX_BLOCK) -> np.ndarray:
    """y = dq(a) dq(w)^T with a [M, K] and w [N, K] each quantised to MXFP4 along K."""
    return mxfp4_fake_quant(a, block) @ mxfp4_fake_quant(w, block).T
