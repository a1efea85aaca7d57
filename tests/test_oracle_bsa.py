"""Pins of the block-sparse attention oracle (CPU only): INT8 codes against
their definition and hand-made midpoints, the keep count, the block
selection on planted structure and against an independent mean-pooling
evaluation, the sparse online softmax against the plain softmax over the
kept keys, and the dense-fallback step rule against the pages' table."""
import math

import numpy as np
import pytest

from oracle import attn_varlen_ref
from oracle.block_sparse_attention import (bsa_attn_emulated_ref, dense_fallback,
                                           int8_quantize_qk_blocks, keep_count,
                                           select_kv_blocks)


def _bf16(a):
    b = np.asarray(a, dtype=np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _qkv(n, heads, d, seed):
    rng = np.random.default_rng(seed)
    return tuple(_bf16(rng.standard_normal((n, heads, d))) for _ in range(3))


def test_int8_codes_definition_and_bounds():
    cu = [0, 100, 100, 229]
    x = _bf16(np.random.default_rng(1).standard_normal((229, 3, 128)) * 3)
    codes, sc = int8_quantize_qk_blocks(x, cu)
    assert sc.dtype == np.float32 and sc.shape == (2 + 3, 3)      # ceil(100/64) + ceil(129/64)
    assert np.abs(codes).max() == 127
    b = 0
    for a, e in [(0, 100), (100, 229)]:
        for t0 in range(a, e, 64):
            t1 = min(e, t0 + 64)
            blk = x[t0:t1]
            amax = np.abs(blk).max(axis=(0, 2))
            # the block's largest magnitude maps to +-127, every code is within
            # half a step of x / (amax / 127) and no other integer is closer
            exact = 127 * blk / amax[None, :, None]
            assert np.all(np.abs(codes[t0:t1] - exact) <= 0.5)
            assert np.all(np.abs(codes[t0:t1]).max(axis=(0, 2)) == 127)
            assert np.array_equal(sc[b], (amax.astype(np.float32) / np.float32(127)))
            b += 1


def test_int8_midpoints_round_to_even_and_zero_blocks():
    # amax = 127: code = round_half_even(x); 2.5 -> 2, 3.5 -> 4, -2.5 -> -2
    x = np.zeros((64, 2, 128))
    x[0, 0, :6] = [127.0, 2.5, 3.5, -2.5, 126.5, 0.5]
    codes, sc = int8_quantize_qk_blocks(x, [0, 64])
    assert list(codes[0, 0, :6]) == [127, 2, 4, -2, 126, 0]
    assert np.all(codes[:, 1] == 0) and sc[0, 1] == 1.0             # all-zero head: scale 1, codes 0


def test_keep_count():
    assert keep_count(10, 0.8) == 2
    assert keep_count(906, 0.8) == 182            # 906 - floor(724.8)
    assert keep_count(1, 0.8) == 1 and keep_count(4, 0.9) == 1
    assert keep_count(7, 0.0) == 7
    assert keep_count(0, 0.5) == 0
    with pytest.raises(ValueError):
        keep_count(5, 1.0)


def test_selection_planted_blocks():
    """Query rows all along e0; key block 5 along e0, block 2 along -e0, the
    rest near zero: with one block kept it is 5, and with all but one kept
    the dropped block is 2."""
    rng = np.random.default_rng(4)
    n = 64 * 8
    q = np.zeros((n, 1, 128))
    q[:, 0, 0] = 1.0
    k = rng.standard_normal((n, 1, 128)) * 0.01
    k[5 * 64:6 * 64, 0, 0] = 2.0
    k[2 * 64:3 * 64, 0, 0] = -2.0
    q8, qs = int8_quantize_qk_blocks(q, [0, n])
    k8, ks = int8_quantize_qk_blocks(k, [0, n])
    sel = select_kv_blocks(q8, qs, k8, ks, [0, n], 0.875)           # keep 1 of 8
    assert all(list(v) == [5] for v in sel.values()) and len(sel) == 2
    sel = select_kv_blocks(q8, qs, k8, ks, [0, n], 0.125)           # keep 7 of 8
    assert all(list(v) == [0, 1, 3, 4, 5, 6, 7] for v in sel.values())


def test_selection_ties_go_to_lower_index_and_short_block_uses_mean():
    """Identical key blocks tie and the lower indices win; a short last block
    competes by its mean, not its sum."""
    n = 64 * 4
    q = np.zeros((n, 1, 128))
    q[:, 0, 0] = 1.0
    k = np.zeros((n, 1, 128))
    k[:, 0, 0] = 1.0
    q8, qs = int8_quantize_qk_blocks(q, [0, n])
    k8, ks = int8_quantize_qk_blocks(k, [0, n])
    sel = select_kv_blocks(q8, qs, k8, ks, [0, n], 0.5)
    assert list(sel[(0, 0)]) == [0, 1]
    m = 64 * 3 + 8
    q = np.zeros((m, 1, 128))
    q[:, 0, 0] = 1.0
    k = np.zeros((m, 1, 128))
    k[:192, 0, 0] = 0.5
    k[192:, 0, 0] = 1.0                 # 8 keys, twice the mean, a sixth of a full block's sum
    q8, qs = int8_quantize_qk_blocks(q, [0, m])
    k8, ks = int8_quantize_qk_blocks(k, [0, m])
    sel = select_kv_blocks(q8, qs, k8, ks, [0, m], 0.75)            # keep 1 of 4
    assert list(sel[(0, 0)]) == [3]


def test_selection_matches_dequantised_block_means():
    """Independent evaluation: rank key blocks by mean(dequantised q over the
    query block) . mean(dequantised k over the key block); where the scores
    are well separated the kept sets agree."""
    cu = [0, 700, 1213]
    heads = 3
    q, k, _ = _qkv(1213, heads, 128, 6)
    k += np.random.default_rng(7).standard_normal((1213 // 64 + 1, heads, 128)).repeat(64, axis=0)[:1213]
    q8, qs = int8_quantize_qk_blocks(q, cu)
    k8, ks = int8_quantize_qk_blocks(k, cu)
    sel = select_kv_blocks(q8, qs, k8, ks, cu, 0.6)

    def deq(codes, sc):
        out = np.zeros(codes.shape)
        b = 0
        for s in range(len(cu) - 1):
            for t0 in range(cu[s], cu[s + 1], 64):
                t1 = min(cu[s + 1], t0 + 64)
                out[t0:t1] = codes[t0:t1] * sc[b].astype(np.float64)[None, :, None]
                b += 1
        return out

    qd, kd = deq(q8, qs), deq(k8, ks)
    checked = 0
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        starts = list(range(a, e, 64))
        for t0 in range(a, e, 256):
            for h in range(heads):
                qm = qd[t0:min(e, t0 + 256), h].mean(axis=0)
                sc = np.array([qm @ kd[j0:min(e, j0 + 64), h].mean(axis=0) for j0 in starts])
                keep = keep_count(len(starts), 0.6)
                srt = np.sort(sc)[::-1]
                if srt[keep - 1] - srt[keep] < 1e-9 * np.abs(srt).max():
                    continue
                assert set(np.argsort(-sc)[:keep]) == set(sel[(h, t0)]), (h, t0)
                checked += 1
    assert checked >= 12


def test_sparsity_zero_unquantised_is_dense_attention():
    cu = [0, 300, 300, 557]
    q, k, v = _qkv(557, 2, 128, 8)
    out, sel = bsa_attn_emulated_ref(q, k, v, cu, 0.0, quantize=False)
    assert all(len(x) == math.ceil(l / 64) for x, l in
               zip([sel[(0, 0)], sel[(0, 300)]], [300, 257]))
    ref = attn_varlen_ref(q, k, v, cu)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sparse_unquantised_is_softmax_over_kept_keys():
    """Plain softmax over the gathered kept keys, written out here."""
    cu = [0, 520, 1000]
    q, k, v = _qkv(1000, 2, 128, 9)
    out, sel = bsa_attn_emulated_ref(q, k, v, cu, 0.7, quantize=False)
    for (h, t0), blocks in sel.items():
        s = 0 if t0 < 520 else 1
        a, e = cu[s], cu[s + 1]
        keys = np.concatenate([np.arange(a + 64 * j, min(e, a + 64 * j + 64)) for j in blocks])
        rows = np.arange(t0, min(e, t0 + 256))
        logits = q[rows, h] @ k[keys, h].T / math.sqrt(128)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        ref = (w / w.sum(axis=1, keepdims=True)) @ v[keys, h]
        assert np.max(np.abs(out[rows, h] - ref)) < 1e-12
        assert len(blocks) == keep_count(math.ceil((e - a) / 64), 0.7)


def test_quantised_sparse_is_close_to_exact_and_dense_when_sparsity_zero():
    cu = [0, 640]
    q, k, v = _qkv(640, 2, 128, 10)
    exact = attn_varlen_ref(q, k, v, cu)
    out, _ = bsa_attn_emulated_ref(q, k, v, cu, 0.0)
    rel = np.linalg.norm(out - exact) / np.linalg.norm(exact)
    assert rel < 5e-2
    # and an exact (quantize=False) sparse run with the same selection is close
    sp, sel = bsa_attn_emulated_ref(q, k, v, cu, 0.5)
    spx, _ = bsa_attn_emulated_ref(q, k, v, cu, 0.5, quantize=False, selection=sel)
    assert np.linalg.norm(sp - spx) / np.linalg.norm(spx) < 5e-2


def test_dense_fallback_window():
    """The pages' 50-step settings: (8, 13) runs 21 dense steps, (8, 12) 20,
    (0, 13) 13, (0, 0) none; start/end are counts, not indices."""
    for start, end, dense in [(8, 13, 21), (8, 12, 20), (0, 13, 13), (0, 0, 0)]:
        flags = [dense_fallback(s, 50, start, end) for s in range(50)]
        assert sum(flags) == dense
        assert all(flags[:start]) and not any(flags[start:50 - end]) and all(flags[50 - end:])


def test_quantised_single_block_matches_direct_formula():
    """With one kept key block the online softmax is one step: written out
    directly from the INT8 / e4m3 definitions (codes and scales recomputed
    here from amax; P = e4m3(448 p) in the numerator, the unquantised p in
    the denominator), the emulation must agree to rounding."""
    from oracle import e4m3_round
    cu = [0, 256]
    q, k, v = _qkv(256, 1, 128, 11)
    out, sel = bsa_attn_emulated_ref(q, k, v, cu, 0.75)            # keep 1 of 4
    (j,) = sel[(0, 0)]
    keys = np.arange(64 * j, 64 * j + 64)
    s_k = np.float64(np.float32(np.abs(k[keys, 0]).max()) / np.float32(127))
    k8 = np.rint(127 * k[keys, 0] / np.abs(k[keys, 0]).max())
    logits = np.zeros((256, 64))
    for b in range(4):
        rows = np.arange(64 * b, 64 * b + 64)
        am = np.abs(q[rows, 0]).max()
        logits[rows] = (np.rint(127 * q[rows, 0] / am) @ k8.T) * np.float64(np.float32(am) / np.float32(127)) * s_k
    logits /= math.sqrt(128)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    vam = np.abs(v[:, 0]).max(axis=0)                                # per channel over the segment
    v8 = e4m3_round(448 * v[keys, 0] / vam[None, :])
    p8 = e4m3_round(448 * p)
    ref = (p8 @ v8) * (vam / 448)[None, :] / (448 * p.sum(axis=1, keepdims=True))
    assert np.max(np.abs(out[:, 0] - ref)) < 1e-12
    # the denominator summed from the encoded P is a different reading
    other = (p8 @ v8) * (vam / 448)[None, :] / p8.sum(axis=1, keepdims=True)
    assert np.max(np.abs(other - ref)) > 1e-6


def test_selection_decides_differences_below_float64_resolution():
    """Scores are compared exactly: two key blocks whose scores differ by
    2^-60 at magnitude 100 (far below float64 resolution) are told apart.
    Q block 0 (scale 1) sums to e_0, Q block 1 (scale 2^-60) to e_1; key
    block 0 sums to 100 e_0, key block 1 to 100 e_0 + e_1, both scales 1, so
    score_0 = 100 and score_1 = 100 + 2^-60. In float64 both are 100.0 and
    the tie would go to block 0; the exact ranking keeps block 1."""
    d = 8
    q8 = np.zeros((128, 1, d), np.int64)
    k8 = np.zeros((128, 1, d), np.int64)
    q8[0, 0, 0] = 1
    q8[64, 0, 1] = 1
    k8[0, 0, 0] = 100
    k8[64, 0, 0] = 100
    k8[64, 0, 1] = 1
    qs = np.array([[1.0], [2.0 ** -60]], np.float32)
    ks = np.array([[1.0], [1.0]], np.float32)
    assert 1.0 * 100 + float(qs[1, 0]) * 0 == 1.0 * 100 + float(qs[1, 0]) * 1      # equal in float64
    sel = select_kv_blocks(q8, qs, k8, ks, [0, 128], 0.5)                          # keep 1 of 2
    assert sel[(0, 0)].tolist() == [1]
    k8[64, 0, 1] = -1                                                              # now 100 - 2^-60
    assert select_kv_blocks(q8, qs, k8, ks, [0, 128], 0.5)[(0, 0)].tolist() == [0]
