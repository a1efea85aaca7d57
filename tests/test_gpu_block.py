"""GPU parity of the whole DiT block (h3_dit_block_forward) against the
float64 oracle, every intermediate tapped, plus bit-exact invariants."""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import announce, bf16_bits_of, compare, to_dev_bf16, to_dev_i32, to_np, torch_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _device_block(ops, dev, inp, split):
    w = {nm: to_dev_bf16(getattr(inp, nm), dev) for nm in ops.WEIGHT_NAMES}
    return ops.DitBlock(w, inp.heads, inp.head_dim, inp.ffn, split)


def _weights_f32(inp):
    return {nm: getattr(inp, nm).f32 for nm in inp.weight_names}


def _run(ops, dev, blk, inp, taps=False):
    cu = inp.cu_seqlens
    n = int(cu[-1])
    tp = blk.make_taps(len(cu) - 1, n, dev) if taps else None
    out = blk.forward(to_dev_bf16(inp.x, dev), to_dev_bf16(inp.cond, dev), to_dev_i32(cu, dev),
                      cu, to_dev_i32(inp.grid, dev), taps=tp)
    return out, tp


# Linear weights use std 0.02 * sqrt(3072 / 512) so that at hidden 512 every
# projection (and the AdaLN gates) has the spread it has at hidden 3072 with
# std 0.02; with plain 0.02 the residual branches would shrink below the bf16
# storage step of the residual stream and could not be checked on their own.
SMALL_STD = 0.02 * (3072 / 512) ** 0.5


def _small_inputs(lens=(300, 0, 211, 65), seed=3, weight_std=SMALL_STD):
    cu = h3synth.cu_from_lengths(list(lens))
    grid = np.zeros((int(cu[-1]), 3), np.int32)
    rng = np.random.default_rng(seed)
    grid[:] = rng.integers(0, 64, size=grid.shape)
    return h3synth.block_inputs(cu, grid, heads=4, head_dim=128, ffn=1024, seed=seed,
                                weight_std=weight_std)


def _magnitudes(ref, x, seg, c, w, eps=1e-6):
    """Local magnitude of each stage's output: to first order, the scale of
    the error that bf16 rounding of the stage's inputs and output can cause.
    For a sum it is the sum of the absolute terms; for a dot product a.W^T it
    is |a|.|W|^T; for silu(g)*u it is |silu(g)|*M_u + max|silu'| * |u| * M_g
    (max |silu'| < 1.1). Computed from the reference's own intermediates."""
    m = oracle.split_modulation(ref["mod"], c)
    n1 = oracle.rmsnorm(x, eps)
    n2 = oracle.rmsnorm(ref["x1"], eps)
    absw = {k: np.abs(np.asarray(v, dtype=np.float64)) for k, v in w.items()}
    h2 = ref["h2"]
    g = h2 @ np.asarray(w["w_gate"], np.float64).T
    u = h2 @ np.asarray(w["w_up"], np.float64).T
    mags = {
        "h": np.abs(n1 * (1 + m["scale1"][seg])) + np.abs(m["shift1"][seg]),
        "x1": np.abs(x) + np.abs(m["gate1"][seg]) * (np.abs(ref["o"]) @ absw["w_o"].T),
        "h2": np.abs(n2 * (1 + m["scale2"][seg])) + np.abs(m["shift2"][seg]),
        "a": (np.abs(oracle.silu(g)) * (np.abs(h2) @ absw["w_up"].T)
              + 1.1 * np.abs(u) * (np.abs(h2) @ absw["w_gate"].T)),
        "x2": np.abs(ref["x1"]) + np.abs(m["gate2"][seg]) * (np.abs(ref["a"]) @ absw["w_down"].T),
    }
    if "h" in ref and "qkv" in ref:
        mags["v"] = np.abs(ref["h"]) @ absw["w_qkv"][2 * c:3 * c].T
    return mags


def _pair_norm(a, heads, d):
    """|(u, v)| of every RoPE pair, repeated over both members (rotation keeps it)."""
    p = a.reshape(a.shape[0], heads, d // 2, 2)
    return np.repeat(np.sqrt((p * p).sum(-1)), 2, axis=-1).reshape(a.shape)


NO_ELEMENTWISE = float("inf")


def _check_block(got, exact, emul, x, seg, c, w, name, heads=None, d=None):
    """Exact oracle: relative Frobenius bar on every stage and on both residual
    branches. Storage-emulating oracle: the elementwise bar with each stage's
    local magnitude (plus the relative Frobenius bar)."""
    keys = [k for k in ("h", "q", "k", "v", "o", "x1", "h2", "a", "x2") if k in got]
    for k in keys:
        compare(got[k], exact[k], f"{name} {k} vs exact", scaled_abs=NO_ELEMENTWISE)
    compare(got["x1"] - x, exact["x1"] - x, f"{name} attention branch x1-x vs exact",
            scaled_abs=NO_ELEMENTWISE)
    compare(got["x2"] - got["x1"], exact["x2"] - exact["x1"],
            f"{name} mlp branch x2-x1 vs exact", scaled_abs=NO_ELEMENTWISE)
    mags = _magnitudes(emul, x, seg, c, w)
    if "q" in got:
        mags["q"] = _pair_norm(emul["q"], heads, d)
        mags["k"] = _pair_norm(emul["k"], heads, d)
    compare(got["h"], exact["h"], f"{name} h vs exact (elementwise)",
            mag=_magnitudes(exact, x, seg, c, w)["h"])
    for k in keys:
        compare(got[k], emul[k], f"{name} {k} vs bf16-storage oracle", mag=mags.get(k))


def test_block_small_all_taps(dev, ops):
    announce("block small (H=4, D=128, C=512, I=1024, 4 segments) all taps")
    inp = _small_inputs()
    split = (32, 48, 48)
    blk = _device_block(ops, dev, inp, split)
    out, tp = _run(ops, dev, blk, inp, taps=True)
    args = (inp.x.f32, inp.cond.f32, _weights_f32(inp), inp.cu_seqlens, inp.grid, 4, 128, split)
    exact = oracle.dit_block_ref(*args)
    emul = oracle.dit_block_ref(*args, emulate_bf16_storage=True)
    c = 512
    compare(to_np(tp["mod"]), exact["mod"], "mod", rel_fro=1e-5, scaled_abs=1e-5)
    qkv = to_np(tp["qkv"])
    got = {"h": to_np(tp["h"]), "q": qkv[:, :c], "k": qkv[:, c:2 * c], "v": qkv[:, 2 * c:],
           "o": to_np(tp["o"]), "x1": to_np(tp["x1"]), "h2": to_np(tp["h2"]),
           "a": to_np(tp["a"]), "x2": to_np(out)}
    seg = oracle.segment_ids(inp.cu_seqlens)
    _check_block(got, exact, emul, inp.x.f32.astype(np.float64), seg, c, _weights_f32(inp),
                 "small", 4, 128)


def test_block_zero_gates_identity_bitwise(dev, ops):
    announce("block with zero gate chunks -> x2 == x")
    inp = _small_inputs(seed=4)
    c = 512
    w_mod = inp.w_mod.bits.copy()
    w_mod[2 * c:3 * c] = 0
    w_mod[5 * c:6 * c] = 0
    inp.w_mod = h3synth.Bf16Array(w_mod, h3synth.bits_to_f32(w_mod))
    blk = _device_block(ops, dev, inp, (32, 48, 48))
    out, _ = _run(ops, dev, blk, inp)
    assert np.array_equal(bf16_bits_of(out), inp.x.bits)


def test_block_deterministic_and_packing_invariant(dev, ops):
    announce("block determinism and packed == per-segment")
    inp = _small_inputs(lens=(300, 211), seed=5)
    blk = _device_block(ops, dev, inp, (32, 48, 48))
    o1 = bf16_bits_of(_run(ops, dev, blk, inp)[0])
    o2 = bf16_bits_of(_run(ops, dev, blk, inp)[0])
    assert np.array_equal(o1, o2)
    cu = inp.cu_seqlens
    for s in range(2):
        a, b = int(cu[s]), int(cu[s + 1])
        sub = h3synth.BlockInputs(np.array([0, b - a], np.int32), inp.grid[a:b],
                                  h3synth.Bf16Array(inp.x.bits[a:b], inp.x.f32[a:b]),
                                  h3synth.Bf16Array(inp.cond.bits[s:s + 1], inp.cond.f32[s:s + 1]),
                                  inp.w_mod, inp.w_qkv, inp.w_o, inp.q_norm, inp.k_norm,
                                  inp.w_gate, inp.w_up, inp.w_down, inp.heads, inp.head_dim,
                                  inp.hidden, inp.ffn, inp.seed)
        alone = bf16_bits_of(_run(ops, dev, blk, sub)[0])
        assert np.array_equal(alone, o1[a:b])


@pytest.mark.parametrize("name,nrows", [("block_10s_58k", 24), ("block_15s_94k", 24)])
def test_block_full_size_sampled_rows(dev, ops, name, nrows):
    """The benchmarked shape and launch; sampled tokens of every stage
    against the exact oracle (keys/values of the whole segment in float64)."""
    announce(f"block {name} full size, {nrows} sampled rows")
    wl = h3synth.WORKLOADS[name]
    inp = h3synth.workload_block_inputs(name)
    split = h3synth.rope_split_for(wl.head_dim)
    blk = _device_block(ops, dev, inp, split)
    out, tp = _run(ops, dev, blk, inp, taps=True)
    n = wl.total_tokens
    rows = np.unique(np.concatenate([h3synth.sample_rows(n, nrows, inp.seed),
                                     [511, 512, 1511, n - 1]]))
    rows = rows[rows < n]
    got = {k: to_np(tp[k][rows]) for k in ("h", "o", "x1", "h2", "a")}
    got["x2"] = to_np(out[rows])
    announce(f"oracle for {len(rows)} rows of {name} (exact, then bf16-storage)")
    args = (inp.x.f32, inp.cond.f32, _weights_f32(inp), inp.cu_seqlens, inp.grid, wl.heads,
            wl.head_dim, split, rows)
    exact = oracle.dit_block_rows_ref(*args)
    emul = oracle.dit_block_rows_ref(*args, emulate_bf16_storage=True)
    seg = oracle.segment_ids(inp.cu_seqlens)[rows]
    _check_block(got, exact, emul, inp.x.f32[rows].astype(np.float64), seg, wl.hidden,
                 _weights_f32(inp), name)
