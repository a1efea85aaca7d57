"""GPU parity of the block with MXFP8 linears (h3_dit_block_forward_mxfp8)
against the float64 oracle with the same MX quantisation of every linear
operand (oracle.dit_block_ref / dit_block_rows_ref with linear_quant), and
against the exact (unquantised) block for the fp8 bar."""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import announce, bf16_bits_of, compare, to_dev_bf16, to_dev_i32, to_np, torch_device

pytestmark = pytest.mark.gpu

REL_MX_EMULATION = 1e-2   # floor of the bar against the MX-emulating oracle (relative Frobenius)
FLOOR_MARGIN = 5e-3       # allowed excess over the emulation's own distance to the exact block
REL_FP8_EXACT = 5e-2      # the fp8 bar, reported: MXFP8 linears alone sit near or above it
NO_ELEMENTWISE = float("inf")
SMALL_STD = 0.02 * (3072 / 512) ** 0.5   # as in the bf16 block tests


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _small_inputs(lens=(300, 0, 211, 65), seed=3):
    cu = h3synth.cu_from_lengths(list(lens))
    grid = np.random.default_rng(seed).integers(0, 64, size=(int(cu[-1]), 3)).astype(np.int32)
    return h3synth.block_inputs(cu, grid, heads=4, head_dim=128, ffn=1024, seed=seed,
                                weight_std=SMALL_STD)


def _block(ops, dev, inp, split):
    w = {nm: to_dev_bf16(getattr(inp, nm), dev) for nm in ops.WEIGHT_NAMES}
    return ops.DitBlockMX(w, inp.heads, inp.head_dim, inp.ffn, split)


def _run(dev, blk, inp):
    cu = inp.cu_seqlens
    return blk.forward(to_dev_bf16(inp.x, dev), to_dev_bf16(inp.cond, dev), to_dev_i32(cu, dev), cu,
                       to_dev_i32(inp.grid, dev))


def _weights(inp):
    return {nm: getattr(inp, nm).f32 for nm in inp.weight_names}


def _relf(a, b) -> float:
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _check_branch(x2, x, emul, emul_alt, exact, name):
    """The residual branch x2 - x.

    A block of MX-quantised linears amplifies tiny differences: a value that
    moves by an ulp can move its E4M3 code by a whole step (1/16), so two
    exact emulations that differ only in whether intermediates are stored in
    bf16 already disagree by several percent. The bar is calibrated on that:
    the GPU may be at most twice as far from the (bf16-storage) emulation as
    the two emulations are from each other, and no further from the exact
    block than the emulation itself plus 5e-3 (the quantisation floor is the
    method's, not the kernels'). A wiring mistake (a wrong modulation chunk,
    scale array or operand) moves the branch by far more than either bound."""
    sens = _relf(emul_alt["x2"] - x, emul["x2"] - x)
    compare(x2 - x, emul["x2"] - x, f"{name} branch x2-x vs MX emulation",
            rel_fro=max(2.0 * sens, REL_MX_EMULATION), scaled_abs=NO_ELEMENTWISE)
    rg, re_ = _relf(x2 - x, exact["x2"] - x), _relf(emul["x2"] - x, exact["x2"] - x)
    print(f"[parity] {name}: emulation sensitivity={sens:.3e}; branch relF gpu-vs-exact={rg:.3e}, "
          f"MX emulation-vs-exact (floor)={re_:.3e}; literal {REL_FP8_EXACT} bar "
          f"{'met' if rg <= REL_FP8_EXACT else 'not met (floor)'}")
    assert rg <= re_ + FLOOR_MARGIN, (rg, re_)


def test_block_mx_small(dev, ops):
    announce("block mx small (H=4, D=128, C=512, I=1024, 4 segments)")
    inp = _small_inputs()
    split = (32, 48, 48)
    out = _run(dev, _block(ops, dev, inp, split), inp)
    args = (inp.x.f32, inp.cond.f32, _weights(inp), inp.cu_seqlens, inp.grid, 4, 128, split)
    emul = oracle.dit_block_ref(*args, emulate_bf16_storage=True, linear_quant=oracle.mx_fake_quant)
    emul_alt = oracle.dit_block_ref(*args, linear_quant=oracle.mx_fake_quant)
    exact = oracle.dit_block_ref(*args)
    _check_branch(to_np(out), inp.x.f32.astype(np.float64), emul, emul_alt, exact, "small")


def test_block_mx_zero_gates_identity_bitwise(dev, ops):
    announce("block mx with zero gate chunks -> x2 == x")
    inp = _small_inputs(seed=4)
    c = 512
    w_mod = inp.w_mod.bits.copy()
    w_mod[2 * c:3 * c] = 0
    w_mod[5 * c:6 * c] = 0
    inp.w_mod = h3synth.Bf16Array(w_mod, h3synth.bits_to_f32(w_mod))
    out = _run(dev, _block(ops, dev, inp, (32, 48, 48)), inp)
    assert np.array_equal(bf16_bits_of(out), inp.x.bits)


def test_block_mx_deterministic(dev, ops):
    announce("block mx determinism")
    inp = _small_inputs(lens=(300, 211), seed=5)
    blk = _block(ops, dev, inp, (32, 48, 48))
    assert np.array_equal(bf16_bits_of(_run(dev, blk, inp)), bf16_bits_of(_run(dev, blk, inp)))


def test_block_mx_full_size_sampled_rows(dev, ops):
    """The benchmarked shape: sampled tokens against the row oracle."""
    name = "block_10s_58k"
    announce(f"block mx {name} full size, sampled rows")
    wl = h3synth.WORKLOADS[name]
    inp = h3synth.workload_block_inputs(name)
    split = h3synth.rope_split_for(wl.head_dim)
    out = _run(dev, _block(ops, dev, inp, split), inp)
    n = wl.total_tokens
    rows = np.unique(np.concatenate([h3synth.sample_rows(n, 8, inp.seed), [511, 512, n - 1]]))
    rows = rows[rows < n]
    got = to_np(out[rows])
    announce(f"oracle for {len(rows)} rows of {name} (MX emulation, then exact)")
    args = (inp.x.f32, inp.cond.f32, _weights(inp), inp.cu_seqlens, inp.grid, wl.heads,
            wl.head_dim, split, rows)
    emul = oracle.dit_block_rows_ref(*args, emulate_bf16_storage=True,
                                     linear_quant=oracle.mx_fake_quant)
    emul_alt = oracle.dit_block_rows_ref(*args, linear_quant=oracle.mx_fake_quant)
    exact = oracle.dit_block_rows_ref(*args)
    _check_branch(got, inp.x.f32[rows].astype(np.float64), emul, emul_alt, exact, name)


def _bsa_attention(sparsity, quantize=True):
    return lambda q, k, v, cu: oracle.bsa_attn_emulated_ref(q, k, v, cu, sparsity, quantize=quantize)[0]


def test_block_mx_bsa_small(dev, ops):
    """The pages' lossy configuration: MXFP8 linears and block-sparse
    INT8/FP8 attention (sparsity 0.5: 3 of 5, 2 of 4 and 1 of 2 key blocks
    kept in the three segments). Against the block emulating both (MX fake
    quantisation, the block-sparse emulation, bf16 storage), with the same
    self-calibrated bar as the MXFP8 block, and against the same block with
    nothing quantised (exact softmax over the kept keys) for the floor."""
    announce("block mx + block-sparse attention small (H=4, D=128, C=512, sparsity 0.5)")
    inp = _small_inputs()
    split = (32, 48, 48)
    w = {nm: to_dev_bf16(getattr(inp, nm), dev) for nm in ops.WEIGHT_NAMES}
    blk = ops.DitBlockMX(w, inp.heads, inp.head_dim, inp.ffn, split, attn_sparsity=0.5)
    out = _run(dev, blk, inp)
    args = (inp.x.f32, inp.cond.f32, _weights(inp), inp.cu_seqlens, inp.grid, 4, 128, split)
    emul = oracle.dit_block_ref(*args, emulate_bf16_storage=True, linear_quant=oracle.mx_fake_quant,
                                attention=_bsa_attention(0.5))
    emul_alt = oracle.dit_block_ref(*args, linear_quant=oracle.mx_fake_quant, attention=_bsa_attention(0.5))
    exact = oracle.dit_block_ref(*args, attention=_bsa_attention(0.5, quantize=False))
    _check_branch(to_np(out), inp.x.f32.astype(np.float64), emul, emul_alt, exact, "small mx+bsa")


def test_block_mx_bsa_deterministic_and_differs_from_dense(dev, ops):
    import torch
    announce("block mx + block-sparse determinism")
    inp = _small_inputs(lens=(600, 211), seed=6)
    w = {nm: to_dev_bf16(getattr(inp, nm), dev) for nm in ops.WEIGHT_NAMES}
    sparse = ops.DitBlockMX(w, inp.heads, inp.head_dim, inp.ffn, (32, 48, 48), attn_sparsity=0.8)
    dense = ops.DitBlockMX(w, inp.heads, inp.head_dim, inp.ffn, (32, 48, 48))
    o1, o2 = _run(dev, sparse, inp), _run(dev, sparse, inp)
    assert np.array_equal(bf16_bits_of(o1), bf16_bits_of(o2))
    assert not np.array_equal(bf16_bits_of(o1), bf16_bits_of(_run(dev, dense, inp)))
