"""Pins of the oracle's varlen attention and bookkeeping (CPU only).

Each check fixes the oracle against something other than itself: a dense
masked brute force written with scalar loops, closed-form special cases,
and invariants of the definition (packed == per segment, rows of the
softmax sum to one).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attn_varlen_ref, schedule_ref, segment_ids, tile_offsets


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _dense_masked_bruteforce(q, k, v, cu, scale):
    """N x N attention with mask seg(i) == seg(j), scalar python loops."""
    n, heads, d = q.shape
    seg = [None] * n
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            seg[t] = s
    out = np.zeros((n, heads, d))
    for h in range(heads):
        for i in range(n):
            logits = []
            for j in range(n):
                if seg[j] != seg[i]:
                    logits.append(None)
                    continue
                acc = 0.0
                for e in range(d):
                    acc += float(q[i, h, e]) * float(k[j, h, e])
                logits.append(acc * scale)
            mx = max(x for x in logits if x is not None)
            w = [0.0 if x is None else math.exp(x - mx) for x in logits]
            tot = sum(w)
            for e in range(d):
                out[i, h, e] = sum(w[j] * float(v[j, h, e]) for j in range(n)) / tot
    return out


def test_attention_equals_dense_masked_bruteforce():
    cu = [0, 5, 5, 12, 13]          # includes an empty and a length-1 segment
    n, heads, d = 13, 2, 8
    q, k, v = _rand((n, heads, d), 1), _rand((n, heads, d), 2), _rand((n, heads, d), 3)
    got = attn_varlen_ref(q, k, v, cu)
    ref = _dense_masked_bruteforce(q, k, v, cu, 1.0 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_packed_equals_per_segment_bitwise():
    lens = [37, 1, 0, 64, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n, heads, d = int(cu[-1]), 3, 16
    q, k, v = _rand((n, heads, d), 4), _rand((n, heads, d), 5), _rand((n, heads, d), 6)
    packed = attn_varlen_ref(q, k, v, cu)
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        alone = attn_varlen_ref(q[a:b], k[a:b], v[a:b], [0, b - a])
        assert np.array_equal(alone, packed[a:b])


def test_softmax_rows_sum_to_one():
    cu = [0, 300, 301, 777]
    n, heads, d = 777, 2, 32
    q, k = 3.0 * _rand((n, heads, d), 7), 3.0 * _rand((n, heads, d), 8)
    v = np.ones((n, heads, d))
    out = attn_varlen_ref(q, k, v, cu)
    assert np.max(np.abs(out - 1.0)) < 1e-12


def test_default_scale_is_inverse_sqrt_head_dim():
    cu = [0, 50]
    q, k, v = _rand((50, 2, 64), 9), _rand((50, 2, 64), 10), _rand((50, 2, 64), 11)
    a = attn_varlen_ref(q, k, v, cu)
    b = attn_varlen_ref(q / 8.0, k, v, cu, scale=1.0)
    assert np.max(np.abs(a - b)) < 1e-13


def test_special_cases():
    heads, d = 2, 16
    # L = 1: the only key is the token itself, o = v
    q, k, v = _rand((1, heads, d), 12), _rand((1, heads, d), 13), _rand((1, heads, d), 14)
    assert np.allclose(attn_varlen_ref(q, k, v, [0, 1]), v, atol=0, rtol=0)
    # identical keys: uniform weights, o = mean of V over the segment
    n = 40
    q = _rand((n, heads, d), 15)
    k = np.repeat(_rand((1, heads, d), 16), n, axis=0)
    v = _rand((n, heads, d), 17)
    out = attn_varlen_ref(q, k, v, [0, n])
    assert np.max(np.abs(out - v.mean(axis=0, keepdims=True))) < 1e-14
    # all value rows equal: o equals that row
    v = np.repeat(_rand((1, heads, d), 18), n, axis=0)
    out = attn_varlen_ref(_rand((n, heads, d), 19), _rand((n, heads, d), 20), v, [0, n])
    assert np.max(np.abs(out - v)) < 1e-14
    # q = lambda * k_j with orthonormal keys: attention collapses onto v_j
    kk = np.linalg.qr(_rand((d, d), 21))[0]          # d orthonormal keys
    k = np.repeat(kk[:, None, :], heads, axis=1)     # [d, H, D]
    v = _rand((d, heads, d), 22)
    j = 5
    q = np.repeat((200.0 * kk[j])[None, None, :], d, axis=0).repeat(heads, axis=1)
    out = attn_varlen_ref(q, k, v, [0, d])
    assert np.max(np.abs(out - v[j][None])) < 1e-12


def test_sampled_rows_equal_full():
    cu = [0, 100, 260]
    q, k, v = _rand((260, 3, 16), 23), _rand((260, 3, 16), 24), _rand((260, 3, 16), 25)
    full = attn_varlen_ref(q, k, v, cu)
    rows = np.array([0, 3, 99, 100, 101, 259])
    part = attn_varlen_ref(q, k, v, cu, rows=rows)
    assert np.array_equal(part, full[rows])


def test_segment_ids_and_tile_offsets_examples():
    assert segment_ids([0, 2, 2, 5]).tolist() == [0, 0, 2, 2, 2]
    assert tile_offsets([0, 2, 2, 131], 128).tolist() == [0, 1, 1, 3]
    assert tile_offsets([0, 128, 256, 257], 128).tolist() == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        segment_ids([1, 3])
    with pytest.raises(ValueError):
        segment_ids([0, 3, 2])


@pytest.mark.parametrize("block_m", [64, 128])
def test_schedule_count_coverage_and_order(block_m):
    lens = [0, 1, 2, 63, 64, 65, 127, 128, 129, 65]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    heads = 3
    items = schedule_ref(cu, heads, block_m)
    assert items.shape == (heads * sum((L + block_m - 1) // block_m for L in lens), 4)
    covered = np.zeros((heads, int(cu[-1])), dtype=int)
    for h, s, q0, qlen in items:
        assert 0 < qlen <= block_m
        assert cu[s] <= q0 and q0 + qlen <= cu[s + 1]
        assert (q0 - cu[s]) % block_m == 0
        covered[h, q0:q0 + qlen] += 1
    assert np.all(covered == 1)
    # order: segments by descending length (ties by index), then head, then tile
    seg_order = []
    for h, s, q0, qlen in items:
        if not seg_order or seg_order[-1] != s:
            seg_order.append(s)
    assert seg_order == [8, 7, 6, 5, 9, 4, 3, 2, 1]
    first = items[items[:, 1] == 8]
    assert first[:, 0].tolist() == sorted(first[:, 0].tolist())


def test_schedule_of_the_tiny_packed_workload():
    items = schedule_ref([0, 704, 1216], 4, 128)
    assert items.shape == (4 * (6 + 4), 4)
    assert items[0].tolist() == [0, 0, 0, 128]
    assert items[5].tolist() == [0, 0, 640, 64]
    assert items[24].tolist() == [0, 1, 704, 128]
    assert items[-1].tolist() == [3, 1, 1088, 128]


def test_rel_frobenius():
    r = np.array([3.0, 4.0])
    assert oracle.rel_frobenius(r + np.array([0.3, 0.4]), r) == pytest.approx(0.1, abs=1e-15)
