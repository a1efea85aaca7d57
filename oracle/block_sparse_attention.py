"""Block-sparse varlen attention with INT8 Q/K and FP8 V, emulated in float64.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline leg may import or call this module; the product path never does.

Source: "MiniMax H3 on Ascend 950PR / 950DT", section "Recommended lossy
configuration (Ascend 950PR / 950DT)": the lossy recipe runs the DiT's
attention as EQBSA, block-sparse attention in mixed precision (Q and K in
INT8, V in FP8) at sparsity 0.8; section "Tuning the EQBSA dense-fallback
window": start_step / end_step count the leading / trailing denoising steps
that run dense attention instead (they are counts, not step indices).

The pages give no block sizes, no block-selection rule and no quantisation
granularity. Readings taken here, each the plainest one the rest supports:
  * INT8 Q and K: symmetric, one scale per (head, 64-token block aligned to
    the segment start), the blocks of the fp8 path. The stored scale is the
    float32 quotient fl32(amax / 127) (1 when amax == 0); the code is
    round-half-even(127 x / amax) of the exact quotient, in [-127, 127].
  * FP8 V: OCP e4m3 with one scale per (segment, head, channel), as in the
    fp8 path (fp8_attention.quantize_v_channels).
  * Blocks: query blocks of 256 rows and key blocks of 64 keys, both aligned
    to the segment start; a query block only sees key blocks of its own
    segment. "Sparsity 0.8" is the fraction of a query block's key blocks
    that are skipped: it keeps keep(n) = max(1, n - floor(n * p / 1000))
    of the segment's n key blocks, p = round(1000 * sparsity).
  * Selection: by the attention logit between block means of the quantised
    Q and K. With Qsum_b[d] the sum of the codes of 64-row Q block b (of the
    query block's up to four), Ksum_j[d] that of key block j, I_bj their
    exact integer dot product, sq_b / sk_j the stored float32 scales and n_j
    the keys in block j, the ranking score is the exact rational
        score_j = (sum over b of sq_b * I_bj) * sk_j / n_j
    (the common positive factors, 1/(query rows) and the softmax scale, are
    dropped: they do not change the ranking). The keep(n) highest scores are
    kept, equal scores going to the lower block index. The ranking is
    computed from float64 estimates with an error bound, and every block
    whose estimate is too close to the keep boundary for the bound to decide
    is ranked again with exact rational arithmetic (fractions.Fraction).
  * Attention over the kept key blocks only, in ascending block order, with
    the fp8 path's online softmax: S = (Q8 . K8) sq sk scale, running row
    max m, p = exp(S - m), P = e4m3(448 p), l the sum of the unquantised p,
    O = (sum P V8) sv / (448 l).
With quantize=False every rounding is the identity (codes are the values,
scales 1) and the result is the exact softmax over the kept keys.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .fp8_attention import E4M3_MAX, e4m3_round, quantize_v_channels

_F = np.float64
I8_MAX = 127
Q_BLOCK = 256
KV_BLOCK = 64
QK_SCALE_BLOCK = 64


def int8_quantize_qk_blocks(x, cu: Sequence[int], block: int = QK_SCALE_BLOCK
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric INT8 codes per (head, segment-aligned `block`-token block).

    x: [N, H, D] (bf16 values). Returns (codes int64 [N, H, D] in [-127, 127],
    scales float32 [num_blocks, H]) with blocks enumerated segment by
    segment. 127 x is exact in float64 for bf16 x, and the quotient by amax
    is either exactly a half-integer (kept exactly, then rounded to even) or
    at least 2^-16 (relative) away from one, far beyond float64 rounding.
    """
    x = np.asarray(x, dtype=_F)
    n, heads, _ = x.shape
    codes = np.zeros(x.shape, dtype=np.int64)
    scales = []
    cu = np.asarray(cu, dtype=np.int64)
    for s in range(cu.size - 1):
        for t0 in range(int(cu[s]), int(cu[s + 1]), block):
            t1 = min(int(cu[s + 1]), t0 + block)
            amax = np.max(np.abs(x[t0:t1]), axis=(0, 2))                          # [H]
            safe = np.where(amax > 0, amax, 1.0)
            q = np.rint(I8_MAX * x[t0:t1] / safe[None, :, None])
            codes[t0:t1] = np.where(amax[None, :, None] > 0, q, 0.0).astype(np.int64)
            sc = np.where(amax > 0, amax.astype(np.float32) / np.float32(I8_MAX), np.float32(1.0))
            scales.append(sc.astype(np.float32))
    sc_arr = np.array(scales, dtype=np.float32).reshape(-1, heads)
    return codes, sc_arr


def keep_count(n_blocks: int, sparsity: float) -> int:
    """Key blocks a query block keeps out of its segment's n_blocks."""
    if not 0.0 <= sparsity < 1.0:
        raise ValueError("sparsity must be in [0, 1)")
    p = int(round(1000.0 * sparsity))
    return max(1, n_blocks - (n_blocks * p) // 1000) if n_blocks > 0 else 0


def _segment_blocks(cu: np.ndarray, size: int):
    """[(segment, first_token, rows)] of the segment-aligned `size`-row blocks."""
    out = []
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for t0 in range(a, b, size):
            out.append((s, t0, min(b, t0 + size) - t0))
    return out


def _exact_scores(qblocks, ksum_i, sk, n_j, idx):
    """Exact rational scores of key blocks `idx`: (sum_b sq_b I_bj) sk_j / n_j."""
    out = {}
    for j in idx:
        tot = Fraction(0)
        for sq, qsum in qblocks:
            tot += Fraction(float(sq)) * int(ksum_i[j] @ qsum)
        out[int(j)] = tot * Fraction(float(sk[j])) / int(n_j[j])
    return out


def select_kv_blocks(q8, q_scale, k8, k_scale, cu: Sequence[int], sparsity: float,
                     query_blocks: Optional[Sequence[Tuple[int, int]]] = None
                     ) -> Dict[Tuple[int, int], np.ndarray]:
    """Kept key blocks of every (head, query block), or of those listed.

    q8, k8: int codes [N, H, D]; q_scale, k_scale: float32 [num_64_blocks, H].
    Returns {(head, first token of the query block): ascending int64 array of
    key-block indices within the segment}.

    Ranking: float64 estimates est_j of the exact scores with a bound e_j on
    their error (each float64 operation adds at most 2^-53 of the running
    magnitude; 2^-46 of the sum of |terms| is used). With K the keep(n)
    leading blocks of the estimate order and R the rest, a block of K whose
    est - e exceeds every est + e of R is in the exact top keep(n) (it beats
    every block of R), and a block of R whose est + e is below every est - e
    of K is not; the blocks left are ranked by their exact scores.
    """
    q8 = np.asarray(q8, dtype=np.int64)
    k8 = np.asarray(k8, dtype=np.int64)
    cu = np.asarray(cu, dtype=np.int64)
    heads = q8.shape[1]
    blocks64 = _segment_blocks(cu, QK_SCALE_BLOCK)
    index64 = {t0: i for i, (_, t0, _) in enumerate(blocks64)}
    if query_blocks is None:
        query_blocks = [(h, t0) for _, t0, _ in _segment_blocks(cu, Q_BLOCK) for h in range(heads)]
    seg_of = {t0: s for s, t0, _ in _segment_blocks(cu, Q_BLOCK)}
    out = {}
    for h, t0 in query_blocks:
        s = seg_of[t0]
        a, b = int(cu[s]), int(cu[s + 1])
        kstarts = list(range(a, b, KV_BLOCK))
        n = len(kstarts)
        ksum = np.stack([k8[j0:min(b, j0 + KV_BLOCK), h].sum(axis=0) for j0 in kstarts])   # [n, D]
        n_j = np.array([min(KV_BLOCK, b - j0) for j0 in kstarts], dtype=np.int64)
        sk = np.array([k_scale[index64[j0], h] for j0 in kstarts], dtype=np.float32)
        qblocks = [(np.float32(q_scale[index64[t], h]), q8[t:min(b, t + QK_SCALE_BLOCK), h].sum(axis=0))
                   for t in range(t0, min(b, t0 + Q_BLOCK), QK_SCALE_BLOCK)]
        acc = np.zeros(n)
        mag = np.zeros(n)
        for sq, qsum in qblocks:
            term = np.float64(sq) * (ksum @ qsum).astype(_F)          # the dot products are exact int64
            acc += term
            mag += np.abs(term)
        est = acc * sk.astype(_F) / n_j
        err = mag * np.abs(sk.astype(_F)) / n_j * 2.0 ** -46
        keep = keep_count(n, sparsity)
        order = np.lexsort((np.arange(n), -est))
        kept, rest = order[:keep], order[keep:]
        if rest.size:
            hi_rest = np.max(est[rest] + err[rest])
            lo_kept = np.min(est[kept] - err[kept])
            if lo_kept <= hi_rest:
                amb = np.concatenate([kept[est[kept] - err[kept] <= hi_rest],
                                      rest[est[rest] + err[rest] >= lo_kept]])
                sure = kept[est[kept] - err[kept] > hi_rest]
                exact = _exact_scores(qblocks, ksum, sk, n_j, amb)
                ranked = sorted(exact, key=lambda j: (-exact[j], j))
                kept = np.concatenate([sure, np.array(ranked[:keep - sure.size], dtype=np.int64)])
        out[(h, t0)] = np.sort(kept).astype(np.int64)
    return out


def bsa_attn_emulated_ref(q, k, v, cu: Sequence[int], sparsity: float,
                          scale: Optional[float] = None, quantize: bool = True,
                          selection: Optional[Dict[Tuple[int, int], np.ndarray]] = None,
                          query_blocks: Optional[Sequence[Tuple[int, int]]] = None):
    """Block-sparse attention emulated in float64 (see module docstring).

    q, k, v: [N, H, D] (bf16 values). `selection` overrides the selection
    (else it is computed from the INT8 codes, also when quantize=False);
    `query_blocks` = [(head, first_token)] restricts the computed blocks.
    Returns (out [N, H, D] float64, rows not computed left 0; selection).
    """
    q = np.asarray(q, dtype=_F)
    k = np.asarray(k, dtype=_F)
    v = np.asarray(v, dtype=_F)
    n, heads, d = q.shape
    cu = np.asarray(cu, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q8, qs = int8_quantize_qk_blocks(q, cu)
    k8, ks = int8_quantize_qk_blocks(k, cu)
    if query_blocks is None:
        query_blocks = [(h, t0) for _, t0, _ in _segment_blocks(cu, Q_BLOCK) for h in range(heads)]
    if selection is None:
        selection = select_kv_blocks(q8, qs, k8, ks, cu, sparsity, query_blocks)
    if quantize:
        qv, kv_ = q8.astype(_F), k8.astype(_F)
        vc, vs = quantize_v_channels(v, cu)
        rnd, p_mul = e4m3_round, E4M3_MAX
        blocks64 = _segment_blocks(cu, QK_SCALE_BLOCK)
        sq_tok = np.zeros((n, heads))
        sk_tok = np.zeros((n, heads))
        for i, (_, t0, r) in enumerate(blocks64):
            sq_tok[t0:t0 + r] = qs[i].astype(_F)
            sk_tok[t0:t0 + r] = ks[i].astype(_F)
    else:
        qv, kv_, vc = q, k, v
        vs = np.ones((cu.size - 1, heads, d))
        rnd, p_mul = (lambda z: z), 1.0
        sq_tok = np.ones((n, heads))
        sk_tok = np.ones((n, heads))
    seg_of = np.zeros(n, dtype=np.int64)
    for s in range(cu.size - 1):
        seg_of[int(cu[s]):int(cu[s + 1])] = s
    out = np.zeros((n, heads, d))
    for h, t0 in query_blocks:
        s = int(seg_of[t0])
        a, b = int(cu[s]), int(cu[s + 1])
        if (t0 - a) % Q_BLOCK:
            raise ValueError("query block must start on a 256-row boundary of its segment")
        rows = np.arange(t0, min(b, t0 + Q_BLOCK))
        qg = qv[rows, h]
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, d))
        for j in selection[(h, t0)]:
            j0 = a + KV_BLOCK * int(j)
            j1 = min(b, j0 + KV_BLOCK)
            sc = (qg @ kv_[j0:j1, h].T) * sq_tok[rows, h][:, None] * sk_tok[j0:j1, h][None, :] * scale
            m_new = np.maximum(m, sc.max(axis=1))
            alpha = np.exp(m - m_new)
            p = np.exp(sc - m_new[:, None])
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + rnd(p_mul * p) @ vc[j0:j1, h]
            m = m_new
        out[rows, h] = acc * vs[s, h][None, :] / (p_mul * l[:, None])
    return out, selection


def dense_fallback(step: int, num_steps: int, start_steps: int, end_steps: int) -> bool:
    """Whether denoising step `step` (0-based, of num_steps) runs dense
    attention: the first start_steps and the last end_steps steps do."""
    if not 0 <= step < num_steps:
        raise ValueError("step out of range")
    return step < start_steps or step >= num_steps - end_steps
