"""GPU parity of the varlen bookkeeping and the bf16 attention kernel.

Every expected value comes from the float64 oracle on the same seeded
inputs; nothing here feeds a device result back into the oracle.
"""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import (announce, bf16_bits_of, compare, to_dev_bf16, to_dev_i32, to_np,
                          torch_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _cu(lens):
    return h3synth.cu_from_lengths(lens)


# --------------------------------------------------------------------------
# bookkeeping: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lens,heads,block_m", [
    ([704, 512], 4, 128),
    ([57960], 24, 128),
    ([93740], 24, 128),
    ([0, 1, 2, 63, 64, 65, 127, 128, 129], 3, 128),
    ([129, 128, 127, 65, 64, 63, 2, 1, 0, 65, 64], 2, 64),
    ([5] * 1500 + [7, 0, 3], 2, 4),
    ([57960], 24, 256),
    ([93740], 24, 256),
    ([32260], 24, 256),
    ([0, 1, 255, 256, 257, 511, 512, 513, 128, 129, 0], 3, 256),
    ([704, 512], 4, 256),
])
def test_bookkeeping_bit_exact(dev, ops, lens, heads, block_m):
    announce(f"bookkeeping lens[:4]={lens[:4]} B={len(lens)} H={heads} BM={block_m}")
    import torch
    cu = _cu(lens)
    seg_id, tile_cu, items = ops.varlen_bookkeeping(to_dev_i32(cu, dev), cu, heads, block_m)
    torch.cuda.synchronize()
    assert np.array_equal(seg_id.cpu().numpy(), oracle.segment_ids(cu))
    assert np.array_equal(tile_cu.cpu().numpy(), oracle.tile_offsets(cu, block_m))
    assert np.array_equal(items.cpu().numpy(), oracle.schedule_ref(cu, heads, block_m))


# --------------------------------------------------------------------------
# attention parity
# --------------------------------------------------------------------------

def _run_attn(ops, dev, inp, heads, head_dim):
    cu = inp.cu_seqlens
    q = to_dev_bf16(inp.q, dev)
    k = to_dev_bf16(inp.k, dev)
    v = to_dev_bf16(inp.v, dev)
    out = ops.attn_varlen(q, k, v, to_dev_i32(cu, dev), cu)
    return out


def test_attention_tiny_packed(dev, ops):
    announce("attention tiny_packed_2req raw q,k,v")
    inp = h3synth.workload_attention_inputs("tiny_packed_2req")
    out = _run_attn(ops, dev, inp, 4, 64)
    ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, inp.cu_seqlens)
    compare(to_np(out), ref, "attn tiny packed")


@pytest.mark.parametrize("head_dim", [64, 128])
def test_attention_ragged_segments(dev, ops, head_dim):
    lens = [1, 63, 64, 65, 0, 127, 129, 300, 1000, 2]
    announce(f"attention ragged D={head_dim} lens={lens}")
    cu = _cu(lens)
    inp = h3synth.attention_inputs(cu, np.zeros((cu[-1], 3), np.int32), 3, head_dim, seed=77)
    out = _run_attn(ops, dev, inp, 3, head_dim)
    ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    compare(to_np(out), ref, f"attn ragged D={head_dim}")


@pytest.mark.parametrize("heads,head_dim", [(8, 64), (16, 128)])
def test_attention_ragged_segments_heads_multiple_of_8(dev, ops, heads, head_dim):
    """With a head count divisible by 8 the kernel hands each XCD the items
    of every eighth head; ragged and empty segments in several sizes."""
    lens = [1, 300, 0, 65, 1000, 64, 257, 0, 2, 513]
    announce(f"attention ragged heads={heads} D={head_dim} lens={lens}")
    cu = _cu(lens)
    inp = h3synth.attention_inputs(cu, np.zeros((cu[-1], 3), np.int32), heads, head_dim, seed=78)
    out = _run_attn(ops, dev, inp, heads, head_dim)
    ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    compare(to_np(out), ref, f"attn ragged heads={heads} D={head_dim}")


def test_attention_length_one_returns_v(dev, ops):
    announce("attention length-1 segments")
    cu = _cu([1, 1, 1, 3, 1])
    inp = h3synth.attention_inputs(cu, np.zeros((cu[-1], 3), np.int32), 2, 128, seed=5)
    out = _run_attn(ops, dev, inp, 2, 128)
    got = bf16_bits_of(out)
    for t in (0, 1, 2, 6):
        assert np.array_equal(got[t], inp.v.bits[t])


def test_attention_empty_is_noop(dev, ops):
    import torch
    announce("attention empty input")
    q = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=dev)
    out = ops.attn_varlen(q, q, q, to_dev_i32([0, 0], dev), [0, 0])
    assert out.shape == (0, 2, 128)


def test_attention_packed_equals_per_segment_bitwise(dev, ops):
    announce("attention packed vs per-segment")
    inp = h3synth.workload_attention_inputs("tiny_packed_2req")
    packed = bf16_bits_of(_run_attn(ops, dev, inp, 4, 64))
    cu = inp.cu_seqlens
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        sub = h3synth.AttnInputs(np.array([0, b - a], np.int32), inp.grid[a:b],
                                 h3synth.Bf16Array(inp.q.bits[a:b], inp.q.f32[a:b]),
                                 h3synth.Bf16Array(inp.k.bits[a:b], inp.k.f32[a:b]),
                                 h3synth.Bf16Array(inp.v.bits[a:b], inp.v.f32[a:b]),
                                 inp.w_q, inp.w_k, inp.seed)
        alone = bf16_bits_of(_run_attn(ops, dev, sub, 4, 64))
        assert np.array_equal(alone, packed[a:b])


def test_attention_deterministic_and_segment_swap(dev, ops):
    announce("attention determinism + equal-length segment swap")
    cu = _cu([300, 300])
    inp = h3synth.attention_inputs(cu, np.zeros((600, 3), np.int32), 2, 128, seed=9)
    o1 = bf16_bits_of(_run_attn(ops, dev, inp, 2, 128))
    o2 = bf16_bits_of(_run_attn(ops, dev, inp, 2, 128))
    assert np.array_equal(o1, o2)
    perm = np.r_[300:600, 0:300]
    sw = h3synth.AttnInputs(cu, inp.grid, *[h3synth.Bf16Array(a.bits[perm], a.f32[perm])
                                            for a in (inp.q, inp.k, inp.v)],
                            inp.w_q, inp.w_k, inp.seed)
    o3 = bf16_bits_of(_run_attn(ops, dev, sw, 2, 128))
    assert np.array_equal(o3, o1[perm])


def test_attention_strided_views_in_packed_qkv(dev, ops):
    """q, k, v as column blocks of one [N, 3*H*D] buffer (the block's layout)."""
    import torch
    announce("attention strided qkv views")
    lens = [200, 77]
    cu = _cu(lens)
    heads, d = 4, 128
    inp = h3synth.attention_inputs(cu, np.zeros((cu[-1], 3), np.int32), heads, d, seed=11)
    n = int(cu[-1])
    qkv = torch.empty((n, 3 * heads * d), dtype=torch.bfloat16, device=dev)
    qkv[:, :heads * d] = to_dev_bf16(inp.q, dev).reshape(n, -1)
    qkv[:, heads * d:2 * heads * d] = to_dev_bf16(inp.k, dev).reshape(n, -1)
    qkv[:, 2 * heads * d:] = to_dev_bf16(inp.v, dev).reshape(n, -1)
    qv = qkv[:, :heads * d].view(n, heads, d)
    kv = qkv[:, heads * d:2 * heads * d].view(n, heads, d)
    vv = qkv[:, 2 * heads * d:].view(n, heads, d)
    out = ops.attn_varlen(qv, kv, vv, to_dev_i32(cu, dev), cu)
    ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    compare(to_np(out), ref, "attn strided views")
    dense = bf16_bits_of(_run_attn(ops, dev, inp, heads, d))
    assert np.array_equal(bf16_bits_of(out), dense)


def test_attention_after_qk_norm_rope_tiny(dev, ops):
    announce("tiny_packed_2req: qk norm+rope then attention")
    inp = h3synth.workload_attention_inputs("tiny_packed_2req")
    cu, grid = inp.cu_seqlens, inp.grid
    q = to_dev_bf16(inp.q, dev)
    k = to_dev_bf16(inp.k, dev)
    v = to_dev_bf16(inp.v, dev)
    split = h3synth.rope_split_for(64)
    ops.qk_rmsnorm_rope(q, k, to_dev_bf16(inp.w_q, dev), to_dev_bf16(inp.w_k, dev),
                        to_dev_i32(grid, dev), split, 1e4, 1e-6)
    qr, kr = oracle.qk_norm_rope_ref(inp.q.f32, inp.k.f32, inp.w_q.f32, inp.w_k.f32, grid,
                                     split, 1e4, 1e-6)
    compare(to_np(q), qr, "q after norm+rope")
    compare(to_np(k), kr, "k after norm+rope")
    out = ops.attn_varlen(q, k, v, to_dev_i32(cu, dev), cu)
    ref = oracle.attn_varlen_ref(qr, kr, inp.v.f32, cu)
    compare(to_np(out), ref, "attn after norm+rope")


def test_attention_5s_32k_sampled_rows(dev, ops):
    """Full 32,260-token, 24 x 128 shape in the benchmarked launch; sampled
    query rows (every head) against the oracle over the whole segment."""
    announce("attention attn_5s_32k full size, sampled rows")
    inp = h3synth.workload_attention_inputs("attn_5s_32k")
    out = _run_attn(ops, dev, inp, 24, 128)
    n = inp.cu_seqlens[-1]
    rows = np.unique(np.concatenate([h3synth.sample_rows(n, 40, inp.seed),
                                     [127, 128, 32255, 32256, 32259]]))
    got = to_np(out)[rows]
    ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, inp.cu_seqlens, rows=rows)
    compare(got, ref, "attn 32k sampled")


# --------------------------------------------------------------------------
# peaked attention: the running max rises after the first key tile, so the
# kernel's lazy rescale (alpha applied to a non-zero O and l) runs
# --------------------------------------------------------------------------

LOG2E = 1.4426950408889634


def _max_rise_log2(q, k, cu, rows=None):
    """Per (row, head): (max logit over the segment) - (max logit over the
    segment's first 64 keys), in log2 units of the softmax argument."""
    n, heads, d = q.shape
    scale = 1.0 / np.sqrt(d)
    rises = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        r = np.arange(a, b) if rows is None else np.array([t for t in rows if a <= t < b])
        if r.size == 0:
            continue
        for h in range(heads):
            lg = (q[r, h].astype(np.float64) @ k[a:b, h].astype(np.float64).T) * scale * LOG2E
            rises.append(lg.max(axis=1) - lg[:, :64].max(axis=1))
    return np.concatenate(rises)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_attention_frame_local_row_max_moves(dev, ops, head_dim):
    """Frame-local inputs: queries gain ~12 nats (17 in log2) with keys of
    their own 1008-token frame, so every query past the first frame meets a
    much larger logit in a later key tile than in the first; the output must
    still meet the bar against the exact oracle."""
    lens = [2600, 0, 1300]
    cu = _cu(lens)
    heads = 2
    announce(f"attention frame-local D={head_dim} lens={lens} (rescale path)")
    inp = h3synth.frame_local_attention_inputs(cu, heads, head_dim, seed=91)
    rise = _max_rise_log2(inp.q.f32, inp.k.f32, cu)
    print(f"[parity] frame-local D={head_dim}: rows with max rise > 16 log2 after tile 0: "
          f"{(rise > 16).mean():.3f}, largest rise {rise.max():.1f}")
    assert (rise > 16).mean() > 0.3
    out = _run_attn(ops, dev, inp, heads, head_dim)
    ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    compare(to_np(out), ref, f"attn frame-local D={head_dim}")


@pytest.mark.parametrize("head_dim", [64, 128])
def test_attention_dominant_key_in_last_tile(dev, ops, head_dim):
    """q = lambda k_j for a key j in the last tile of a 1,100-token segment
    (and of a second, ragged segment): the logit of j rises some 30 log2
    units above everything seen before, so the rescale runs on the last tile
    with O and l already accumulated over 17 tiles; the output tends to
    v_j and must meet the bar elementwise against the exact oracle."""
    lens = [1100, 1037]
    cu = _cu(lens)
    heads = 2
    n = int(cu[-1])
    announce(f"attention dominant key in the last tile D={head_dim} lens={lens}")
    inp = h3synth.attention_inputs(cu, np.zeros((n, 3), np.int32), heads, head_dim, seed=93)
    q = inp.q.f32.copy()
    rng = np.random.default_rng(94)
    for s, j_off in ((0, 1090), (1, 1030)):
        a = int(cu[s])
        j = a + j_off
        rows = a + rng.choice(lens[s], size=lens[s] // 2, replace=False)
        for h in range(heads):
            kj = inp.k.f32[j, h].astype(np.float64)
            lam = 21.0 * np.sqrt(head_dim) / float(kj @ kj)   # q . k_j / sqrt(D) ~ 21 nats
            q[rows, h] = (lam * kj).astype(np.float32)
    qb = h3synth.Bf16Array.from_f32(q)
    rise = _max_rise_log2(qb.f32, inp.k.f32, cu)
    print(f"[parity] dominant key D={head_dim}: rows with max rise > 16 log2: {(rise > 16).mean():.3f}")
    assert (rise > 16).mean() > 0.3
    inp2 = h3synth.AttnInputs(cu, inp.grid, qb, inp.k, inp.v, inp.w_q, inp.w_k, inp.seed)
    out = _run_attn(ops, dev, inp2, heads, head_dim)
    ref = oracle.attn_varlen_ref(qb.f32, inp.k.f32, inp.v.f32, cu)
    compare(to_np(out), ref, f"attn dominant last-tile key D={head_dim}")
