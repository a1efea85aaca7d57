"""Float64 emulation of fp8 (e4m3) varlen attention with skip-softmax.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline leg may import or call this module; the product path never does.

Sources, cited by page title and section:
  [FastH3-EN] "MiniMax H3 FastH3 real-time serving with vLLM-Omni", section
      "Scaling beyond the FastH3 profile", bullet "Sparse & quantized
      attention": SAGE runs attention in FP8; Skip-Softmax skips work for
      unimportant parts of the softmax.
  [FastH3-ZH] "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长", section
      "其他加速路径：有损但可控" (lossy paths): SAGE quantises the attention
      computation to FP8; Skip-Softmax dynamically skips unimportant Softmax
      and P x V work (the Q K^T product is still computed).

The pages do not give the quantisation granularity, the P encoding or the
skip threshold. This module follows this reading:
  * format: OCP e4m3fn (max 448, subnormals down to 2^-9), round to nearest
    even, saturating; scale = amax / 448 (1 when amax == 0); the code of x is
    e4m3(x / scale) with the scale taken exactly, i.e. RNE(448 x / amax);
  * Q and K: one scale per (head, 64-token block), blocks aligned to the
    segment start (the last block of a segment may be short);
  * V: one scale per (segment, head, channel), so it factors out of the sum
    over keys and is applied once at the end;
  * P: e4m3(448 * p) with p = exp(s - m) relative to the running row max
    feeds the P x V product; the softmax denominator l is the sum of the
    unquantised p (only the operands of the two products are encoded; the
    row sum is an accumulation, kept at full precision like the products'
    accumulators);
  * tiles: keys in blocks of 64 from the segment start, in ascending order,
    online softmax across them;
  * skip rule: a key tile is skipped for a group of query rows iff it is not
    the segment's first key tile and, for every valid row r of the group, the
    largest logit of r over the tile's valid keys is below m_r - threshold
    (natural-log units, m_r the running max before the tile). A skipped tile
    contributes nothing (no exp, no P x V) to those rows.

This is an approximation of exact attention: the exact result is in
h3_oracle.attn_varlen_ref, and this module reproduces the quantisation grid
and tile order of the fp8 kernel so that the kernel can be compared to it
tightly.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

_F = np.float64
E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANTISSA_BITS = 3


def e4m3_round(a) -> np.ndarray:
    """Round to the nearest OCP e4m3fn value (ties to even), saturating at +-448.

    The spacing of representable magnitudes in [2^e, 2^(e+1)) is 2^(e-3) for
    e >= -6; below 2^-6 the spacing stays 2^-9 (subnormals).
    """
    a = np.asarray(a, dtype=_F)
    mag = np.abs(a)
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** E4M3_MIN_NORMAL_EXP)))
    ulp = np.power(2.0, e - E4M3_MANTISSA_BITS)
    r = np.round(mag / ulp) * ulp            # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, a)


def _amax_scale(block: np.ndarray, axis=None) -> Tuple[np.ndarray, np.ndarray]:
    """(amax, scale): scale = amax / 448, or 1 where amax == 0."""
    amax = np.max(np.abs(block), axis=axis)
    return amax, np.where(amax > 0, amax / E4M3_MAX, 1.0)


def _codes(x: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """e4m3(x / scale) with scale = amax / 448 taken exactly: the code is
    RNE(448 x / amax), evaluated without rounding the scale first (zero where
    amax == 0). For bf16 inputs 448 x is exact and the one division decides
    exactly: a quotient that is exactly a rounding midpoint stays one and
    goes to the even code, any other is at least 2^-12 (relative) away from
    one, far beyond the division's rounding."""
    den = np.where(amax > 0, amax, 1.0)
    return e4m3_round(E4M3_MAX * x / den)


def quantize_qk_blocks(x, cu: Sequence[int], block: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Per (head, segment-aligned `block`-token block) quantisation of q or k.

    x: [N, H, D]. Returns (codes as float64 values on the e4m3 grid [N, H, D],
    scales [num_blocks, H]) with blocks enumerated segment by segment.
    """
    x = np.asarray(x, dtype=_F)
    n, heads, _ = x.shape
    codes = np.zeros_like(x)
    scales = []
    cu = np.asarray(cu, dtype=np.int64)
    for s in range(cu.size - 1):
        for t0 in range(int(cu[s]), int(cu[s + 1]), block):
            t1 = min(int(cu[s + 1]), t0 + block)
            amax, sc = _amax_scale(x[t0:t1], axis=(0, 2))          # [H]
            codes[t0:t1] = _codes(x[t0:t1], amax[None, :, None])
            scales.append(sc)
    sc_arr = np.array(scales, dtype=_F).reshape(-1, heads)
    return codes, sc_arr


def quantize_v_channels(v, cu: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Per (segment, head, channel) quantisation of v: codes [N,H,D], scales [B,H,D]."""
    v = np.asarray(v, dtype=_F)
    n, heads, d = v.shape
    cu = np.asarray(cu, dtype=np.int64)
    codes = np.zeros_like(v)
    scales = np.ones((cu.size - 1, heads, d), dtype=_F)
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        amax, sc = _amax_scale(v[a:b], axis=0)                       # [H, D]
        codes[a:b] = _codes(v[a:b], amax[None])
        scales[s] = sc
    return codes, scales


def _block_scale_per_token(scales: np.ndarray, cu: Sequence[int], block: int) -> np.ndarray:
    """Expand [num_blocks, H] block scales to [N, H] per token."""
    cu = np.asarray(cu, dtype=np.int64)
    out = []
    b = 0
    for s in range(cu.size - 1):
        for t0 in range(int(cu[s]), int(cu[s + 1]), block):
            t1 = min(int(cu[s + 1]), t0 + block)
            out.append(np.repeat(scales[b][None, :], t1 - t0, axis=0))
            b += 1
    heads = scales.shape[1] if scales.ndim == 2 else 0
    return np.concatenate(out, axis=0) if out else np.zeros((0, heads), _F)


def fp8_attn_emulated_ref(q, k, v, cu: Sequence[int], scale: Optional[float] = None,
                          block_n: int = 64, qk_block: int = 64, group_rows: int = 32,
                          group_origin: int = 128, skip: bool = False,
                          threshold: float = 8.0, quantize: bool = True,
                          groups: Optional[Sequence[Tuple[int, int]]] = None):
    """fp8 attention emulated in float64 (see module docstring).

    Query rows are processed in groups of `group_rows` consecutive tokens;
    groups start at multiples of `group_rows` inside query tiles of
    `group_origin` rows that start at the segment start (the kernel's query
    tile), so a group never spans two segments. With `groups` = [(head,
    first_token)], only those groups are computed.

    Returns (out [N, H, D] float64 (rows not computed stay 0),
             skipped [list of (head, first_token, skipped_tiles, tiles)]).
    With quantize=False every rounding step is the identity, which leaves the
    plain tiled online softmax (used to pin the tiling against the exact
    definition).
    """
    q = np.asarray(q, dtype=_F)
    k = np.asarray(k, dtype=_F)
    v = np.asarray(v, dtype=_F)
    n, heads, d = q.shape
    cu = np.asarray(cu, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rnd = e4m3_round if quantize else (lambda z: np.asarray(z, dtype=_F))
    if quantize:
        qc, qs = quantize_qk_blocks(q, cu, qk_block)
        kc, ks = quantize_qk_blocks(k, cu, qk_block)
        vc, vs = quantize_v_channels(v, cu)
        sq_tok = _block_scale_per_token(qs, cu, qk_block)   # [N, H]
        sk_tok = _block_scale_per_token(ks, cu, qk_block)
        p_mul = E4M3_MAX
    else:
        qc, kc, vc = q, k, v
        sq_tok = np.ones((n, heads), _F)
        sk_tok = np.ones((n, heads), _F)
        vs = np.ones((cu.size - 1, heads, d), _F)
        p_mul = 1.0

    seg_of = np.zeros(n, dtype=np.int64)
    for s in range(cu.size - 1):
        seg_of[int(cu[s]):int(cu[s + 1])] = s

    if groups is None:
        groups = []
        for s in range(cu.size - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            for h in range(heads):
                for t0 in range(a, b, group_rows):
                    groups.append((h, t0))

    out = np.zeros((n, heads, d), dtype=_F)
    report = []
    for h, t0 in groups:
        s = int(seg_of[t0])
        a, b = int(cu[s]), int(cu[s + 1])
        if (t0 - a) % group_rows != 0 and (t0 - a) % group_origin != 0:
            raise ValueError("group must start on a group boundary of its segment")
        t1 = min(b, t0 + group_rows, a + ((t0 - a) // group_origin + 1) * group_origin)
        rows = np.arange(t0, t1)
        qg = qc[rows, h, :]
        sq = sq_tok[rows, h]
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, d))
        ntiles = 0
        nskip = 0
        for j0 in range(a, b, block_n):
            j1 = min(b, j0 + block_n)
            ntiles += 1
            sc = (qg @ kc[j0:j1, h, :].T) * sq[:, None] * sk_tok[j0:j1, h][None, :] * scale
            tmax = sc.max(axis=1)
            if skip and j0 > a and np.all(tmax < m - threshold):
                nskip += 1
                continue
            m_new = np.maximum(m, tmax)
            alpha = np.exp(m - m_new)
            p = np.exp(sc - m_new[:, None])
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + rnd(p_mul * p) @ vc[j0:j1, h, :]
            m = m_new
        out[rows, h, :] = acc * vs[s, h][None, :] / (p_mul * l[:, None])
        report.append((h, t0, nskip, ntiles))
    return out, report
