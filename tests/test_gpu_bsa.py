"""GPU parity of block-sparse attention with INT8 Q/K and FP8 V
(h3_attn_block_sparse): the kept-block lists bit for bit against the
oracle's exact selection (the kernel ranks float64 scores, which can only
differ from the exact ranking on scores within float64 rounding of each
other at the keep boundary; none occur in these inputs), the output against the float64 emulation at the 1e-2 bar, and
against the exact softmax over the same kept keys with the emulation's own
distance as the floor (5e-3 margin), the literal 5e-2 outcome printed."""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import announce, compare, to_dev_bf16, to_dev_i32, to_np, torch_device

pytestmark = pytest.mark.gpu

REL_FP8_EXACT = 5e-2
FLOOR_MARGIN = 5e-3
# elementwise bar against the emulation: the fp8 bar (5e-2 of max(1, |ref|));
# the kernel's softmax denominator is the sum of the encoded P, the
# emulation's the sum of the unquantised p, which moves single outputs of
# peaked rows by up to about 2 % (relative Frobenius error held to 1e-2)
SCALED_ABS_FP8 = 5e-2
D = 128


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _run(ops, dev, inp, sparsity):
    import torch
    cu = inp.cu_seqlens
    heads = inp.q.bits.shape[1]
    lists = torch.full((heads, ops.fp8_num_tiles(cu), ops.attn_block_sparse_list_stride(cu, sparsity)),
                       -1, dtype=torch.int32, device=dev)
    out = ops.attn_block_sparse(to_dev_bf16(inp.q, dev), to_dev_bf16(inp.k, dev), to_dev_bf16(inp.v, dev),
                                to_dev_i32(cu, dev), cu, sparsity=sparsity, kv_block_lists=lists)
    return out, lists.cpu().numpy()


def _tile_index(cu):
    idx, t = {}, 0
    for s in range(len(cu) - 1):
        for t0 in range(int(cu[s]), int(cu[s + 1]), 64):
            idx[t0] = t
            t += 1
    return idx


def _check_lists(lists, sel, cu, heads_map=None):
    tidx = _tile_index(cu)
    for (h, t0), blocks in sel.items():
        row = lists[h if heads_map is None else heads_map[h], tidx[t0]]
        assert np.array_equal(row[:len(blocks)], blocks), (h, t0, row[:len(blocks)], blocks)
        assert np.all(row[len(blocks):] == -1), (h, t0)          # nothing written past keep


def _relf(a, b) -> float:
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _check_output(got, q, k, v, cu, sparsity, name, query_blocks=None, mask=None):
    emu, sel = oracle.bsa_attn_emulated_ref(q, k, v, cu, sparsity, query_blocks=query_blocks)
    exact, _ = oracle.bsa_attn_emulated_ref(q, k, v, cu, sparsity, quantize=False, selection=sel,
                                            query_blocks=query_blocks)
    if mask is not None:
        got, emu, exact = (np.where(mask, a, 0.0) for a in (got, emu, exact))
    assert np.all(np.isfinite(got))
    compare(got, emu, f"{name} vs emulation", scaled_abs=SCALED_ABS_FP8)
    rg, re_ = _relf(got, exact), _relf(emu, exact)
    print(f"[parity] {name}: relF gpu-vs-exact-sparse={rg:.3e} emulation-vs-exact (floor)={re_:.3e} "
          f"literal 5e-2 bar {'met' if rg <= REL_FP8_EXACT else 'not met (floor)'}")
    assert rg <= re_ + FLOOR_MARGIN, (rg, re_)
    return sel


@pytest.mark.parametrize("sparsity", [0.0, 0.6, 0.8])
def test_bsa_multi_segment(dev, ops, sparsity):
    heads = 3
    lens = [700, 0, 513]
    cu = h3synth.cu_from_lengths(lens)
    announce(f"bsa lens={lens} H={heads} sparsity={sparsity}")
    inp = h3synth.attention_inputs(cu, np.zeros((int(cu[-1]), 3), np.int32), heads, D, seed=501)
    out, lists = _run(ops, dev, inp, sparsity)
    sel = _check_output(to_np(out), inp.q.f32, inp.k.f32, inp.v.f32, cu, sparsity, f"bsa s={sparsity}")
    _check_lists(lists, sel, cu)


def test_bsa_short_segments_keep_one(dev, ops):
    """Segments of 1..65 tokens keep a single block; ragged last key blocks."""
    heads = 2
    lens = [1, 63, 64, 65, 0, 300]
    cu = h3synth.cu_from_lengths(lens)
    announce(f"bsa short segments lens={lens}")
    inp = h3synth.attention_inputs(cu, np.zeros((int(cu[-1]), 3), np.int32), heads, D, seed=502)
    out, lists = _run(ops, dev, inp, 0.8)
    sel = _check_output(to_np(out), inp.q.f32, inp.k.f32, inp.v.f32, cu, 0.8, "bsa short segments")
    _check_lists(lists, sel, cu)


def test_bsa_frame_local(dev, ops):
    """Frame-local inputs (queries prefer keys of their own 1008-token frame):
    the selection is structured, the output still within the bar."""
    heads = 2
    cu, _ = h3synth.pack([h3synth.Request(64, 128, 3), h3synth.Request(32, 96, 2)])
    announce(f"bsa frame-local cu={cu.tolist()}")
    inp = h3synth.frame_local_attention_inputs(cu, heads, D, seed=503)
    out, lists = _run(ops, dev, inp, 0.8)
    sel = _check_output(to_np(out), inp.q.f32, inp.k.f32, inp.v.f32, cu, 0.8, "bsa frame-local")
    _check_lists(lists, sel, cu)
    # the kept blocks concentrate on the query's own frame
    own = tot = 0
    for (h, t0), blocks in sel.items():
        s = int(np.searchsorted(cu, t0, side="right") - 1)
        frame = t0 // 1008
        own += sum(1 for j in blocks if (int(cu[s]) + 64 * int(j)) // 1008 == frame)
        tot += len(blocks)
    assert own > 0.5 * tot


def test_bsa_deterministic(dev, ops):
    import torch
    cu = h3synth.cu_from_lengths([900, 400])
    inp = h3synth.attention_inputs(cu, np.zeros((1300, 3), np.int32), 2, D, seed=504)
    o1, l1 = _run(ops, dev, inp, 0.8)
    o2, l2 = _run(ops, dev, inp, 0.8)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert np.array_equal(l1, l2)


def test_bsa_full_size_sampled_blocks(dev, ops):
    """57,960 tokens, 24 heads, sparsity 0.8: the whole pass on the GPU (the
    launch the bench times); sampled (head, query block) pairs: their lists
    bit for bit, their outputs against the emulation and the exact sparse
    softmax (the oracle quantises the two sampled heads only: scales are per
    head)."""
    import torch
    w = h3synth.WORKLOADS["attn_fp8_10s_58k"]
    inp = h3synth.workload_attention_inputs(w.name)
    cu = inp.cu_seqlens
    n = int(cu[-1])
    announce(f"bsa full size N={n} H={w.heads} sparsity=0.8")
    out, lists = _run(ops, dev, inp, 0.8)
    hs = [5, 20]
    rng = np.random.default_rng(505)
    nq = (n + 255) // 256
    starts = sorted({0, 256 * (nq - 1)} | set((256 * rng.integers(0, nq, 4)).tolist()))
    qblocks = [(i % 2, t0) for i, t0 in enumerate(starts)]
    q, k, v = (a.f32[:, hs] for a in (inp.q, inp.k, inp.v))
    rows = np.array(sorted({t for _, t0 in qblocks for t in range(t0, min(n, t0 + 256))}))
    got = np.zeros((n, 2, D))
    got[rows] = to_np(out.index_select(0, torch.from_numpy(rows).to(dev))[:, hs])
    mask = np.zeros((n, 2, 1), dtype=bool)
    for hi, t0 in qblocks:
        mask[t0:min(n, t0 + 256), hi] = True
    sel = _check_output(got, q, k, v, cu, 0.8, "bsa 58k sampled", query_blocks=qblocks, mask=mask)
    _check_lists(lists, sel, cu, heads_map={0: hs[0], 1: hs[1]})
    assert all(len(b) == oracle.keep_count((n + 63) // 64, 0.8) for b in sel.values())


def test_bsa_maximum_segment(dev, ops):
    """The largest segment the path takes: 262,144 tokens = 4096 key blocks
    (the selection sorts 4096 pairs in LDS), one head, sparsity 0.9 (410
    kept). Lists of four sampled query blocks bit for bit, their outputs
    against the emulation."""
    import torch
    n = 4096 * 64
    cu = np.array([0, n], np.int32)
    announce(f"bsa maximum segment N={n} H=1 sparsity=0.9")
    inp = h3synth.attention_inputs(cu, np.zeros((n, 3), np.int32), 1, D, seed=506)
    out, lists = _run(ops, dev, inp, 0.9)
    qblocks = [(0, 0), (0, 256 * 417), (0, 256 * 700), (0, n - 256)]
    rows = np.array(sorted({t for _, t0 in qblocks for t in range(t0, t0 + 256)}))
    got = np.zeros((n, 1, D))
    got[rows] = to_np(out.index_select(0, torch.from_numpy(rows).to(dev)))
    mask = np.zeros((n, 1, 1), dtype=bool)
    mask[rows] = True
    sel = _check_output(got, inp.q.f32, inp.k.f32, inp.v.f32, cu, 0.9, "bsa max segment",
                        query_blocks=qblocks, mask=mask)
    _check_lists(lists, sel, cu)
    assert all(len(b) == 410 for b in sel.values())


def test_bsa_empty_and_rejected(dev, ops):
    """No tokens: nothing launched, success. One token over the maximum
    segment: H3_ERR_UNSUPPORTED before any launch."""
    import torch
    from audio_diffusion_transformer_packed_amd import _lib as L
    z = torch.empty((0, 2, D), dtype=torch.bfloat16, device=dev)
    cu = np.array([0, 0], np.int32)
    out = ops.attn_block_sparse(z, z, z, to_dev_i32(cu, dev), cu, sparsity=0.8)
    assert out.shape == (0, 2, D)
    n = 4096 * 64 + 1
    cu = np.array([0, n], np.int32)
    q = torch.zeros((n, 1, D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(Exception) as e:
        ops.attn_block_sparse(q, q, q, to_dev_i32(cu, dev), cu, sparsity=0.8)
    assert "262144" in str(e.value) or str(L.H3_ERR_UNSUPPORTED) in str(e.value) or "UNSUPPORTED" in str(e.value)


def test_bsa_ties_go_to_lower_blocks(dev, ops):
    """Equal scores: head 0 has all-zero queries (every score 0), head 1 keys
    that repeat every 64 tokens (every full block scores the same). The GPU
    lists must break the ties to the lower block index, as the oracle does;
    the outputs must still match the emulation."""
    lens = [64 * 12, 64 * 7 + 9]
    cu = h3synth.cu_from_lengths(lens)
    n = int(cu[-1])
    announce(f"bsa ties lens={lens}")
    inp = h3synth.attention_inputs(cu, np.zeros((n, 3), np.int32), 2, D, seed=507)
    q_bits, k_bits = inp.q.bits.copy(), inp.k.bits.copy()
    q_bits[:, 0] = 0
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        for t in range(a + 64, b):
            k_bits[t, 1] = k_bits[a + (t - a) % 64, 1]
    inp.q = h3synth.Bf16Array(q_bits, h3synth.bits_to_f32(q_bits))
    inp.k = h3synth.Bf16Array(k_bits, h3synth.bits_to_f32(k_bits))
    out, lists = _run(ops, dev, inp, 0.75)
    sel = _check_output(to_np(out), inp.q.f32, inp.k.f32, inp.v.f32, cu, 0.75, "bsa ties")
    _check_lists(lists, sel, cu)
    for (h, t0), blocks in sel.items():
        if h == 0:
            assert list(blocks) == list(range(len(blocks)))
