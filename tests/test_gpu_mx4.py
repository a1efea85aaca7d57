"""GPU parity of the MXFP4 linears and block against the float64 MXFP4
emulation (oracle.mx_linear: OCP MX v1.0 MXFP4, E2M1 elements): quantisation
codes and scales bit for bit, the GEMMs at the bf16 output bar, the block
against the storage-emulating MXFP4 block with a self-calibrated bar."""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import announce, bf16_bits_of, compare, to_dev_bf16, to_dev_i32, to_np, torch_device

pytestmark = pytest.mark.gpu

NO_ELEMENTWISE = float("inf")
REL_MX_EMULATION = 1e-2
FLOOR_MARGIN = 5e-3
SMALL_STD = 0.02 * (3072 / 512) ** 0.5


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _unpack(mx4):
    """(codes [rows, k] 4-bit, exponents [rows, k/32]) from the device layouts."""
    packed = mx4.codes.cpu().numpy()
    rows, half = packed.shape
    k = 2 * half
    codes = np.empty((rows, k), np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    s = mx4.scales.cpu().numpy().astype(np.int64)
    j = np.arange(k // 32)[None, :]
    r = np.arange(rows)[:, None]
    e = s[((j // 8) * rows + r) * 8 + (j % 2) * 4 + (j % 8) // 2] - 127
    return codes, e


def _mixed(rows, k, seed):
    """bf16 values with per-block magnitudes over 10^[-4, 4], some all-zero
    blocks, blocks whose maximum saturates (just below 8 times a power of
    two), blocks with exact E2M1 midpoints, signed zeros and subnormals."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k))
    x *= np.power(10.0, rng.uniform(-4, 4, size=(rows, k // 32))).repeat(32, axis=1)
    nb = rows * k // 32
    blocks = x.reshape(nb, 32)
    zero = rng.random(nb) < 0.05
    blocks[zero] = 0.0
    blocks[zero, 3] = -0.0
    sat = rng.random(nb) < 0.05
    blocks[sat, 0] = np.sign(blocks[sat, 0] + 0.5) * 7.9 * np.power(2.0, rng.integers(-20, 20, size=sat.sum()))
    mid = rng.random(nb) < 0.05
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    blocks[mid] = rng.choice(mids, size=(mid.sum(), 32)) * rng.choice([-1.0, 1.0], size=(mid.sum(), 32))
    blocks[mid, 0] = 6.0                                    # amax 6: scale 1, the midpoints stay exact
    sub = rng.random(nb) < 0.02
    blocks[sub] = rng.standard_normal((sub.sum(), 32)) * 2.0 ** -130
    return h3synth.Bf16Array.from_f32(x.astype(np.float32))


@pytest.mark.parametrize("rows,k,pad", [(1, 256, 0), (37, 512, 32), (300, 768, 0)])
def test_mx4_quantize_bit_exact(dev, ops, rows, k, pad):
    announce(f"mxfp4 quantize rows={rows} k={k} row pad={pad}")
    x = _mixed(rows, k + pad, 700 + rows)
    mx = ops.mx4_quantize(to_dev_bf16(x, dev)[:, :k])
    codes, e = _unpack(mx)
    want_codes, want_e = oracle.mxfp4_codes(x.f32.astype(np.float64)[:, :k])
    assert np.array_equal(e, want_e)
    assert np.array_equal(codes, want_codes)


def _pair(ops, dev, m, n, k, seed):
    a = _mixed(m, k, seed)
    w = h3synth.Bf16Array.from_f32((np.random.default_rng(seed + 1).standard_normal((n, k)) * 0.02)
                                   .astype(np.float32))
    return a, w, ops.mx4_quantize(to_dev_bf16(a, dev)), ops.mx4_quantize(to_dev_bf16(w, dev))


@pytest.mark.parametrize("m,n,k", [(1, 8, 256), (300, 264, 512), (513, 384, 768), (256, 256, 3072)])
def test_linear_mx4_store(dev, ops, m, n, k):
    announce(f"linear mxfp4 m={m} n={n} k={k}")
    a, w, am, wm = _pair(ops, dev, m, n, k, 710 + m)
    y = ops.linear_mx4(am, wm)
    ref = oracle.mxfp4_linear_ref(a.f32, w.f32)
    # block magnitudes span 10^[-4, 4]: an output's rounding error scales
    # with the sum of its terms' magnitudes, not with its (cancelled) value
    mag = np.abs(oracle.mxfp4_fake_quant(a.f32)) @ np.abs(oracle.mxfp4_fake_quant(w.f32)).T
    compare(to_np(y), ref, f"linear mxfp4 m={m} n={n} k={k}", mag=mag)


@pytest.mark.parametrize("m,n,k", [(333, 256, 512), (600, 128, 768)])
def test_linear_swiglu_mx4(dev, ops, m, n, k):
    announce(f"linear swiglu mxfp4 m={m} n={n} k={k}")
    rng = np.random.default_rng(720 + m)
    a = h3synth.Bf16Array.from_f32(rng.standard_normal((m, k)).astype(np.float32))
    wg = h3synth.Bf16Array.from_f32((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    wu = h3synth.Bf16Array.from_f32((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    q = lambda t: ops.mx4_quantize(to_dev_bf16(t, dev))
    y = ops.linear_swiglu_mx4(q(a), q(wg), q(wu))
    fq = oracle.mxfp4_fake_quant
    aq, gq, uq = fq(a.f32), fq(wg.f32), fq(wu.f32)
    ref = oracle.swiglu_ref(aq, gq, uq)
    g, u = aq @ gq.T, aq @ uq.T
    tg, tu = np.abs(aq) @ np.abs(gq).T, np.abs(aq) @ np.abs(uq).T
    mag = np.abs(oracle.silu(g)) * tu + 1.1 * np.abs(u) * tg
    compare(to_np(y), ref, f"swiglu mxfp4 m={m} n={n} k={k}", mag=mag)


def test_linear_gated_residual_mx4_multi_segment(dev, ops):
    import torch
    announce("linear gated residual mxfp4, 3 segments")
    lens = [100, 0, 157, 300]
    cu = h3synth.cu_from_lengths(lens)
    m, n, k = int(cu[-1]), 392, 512
    a, w, am, wm = _pair(ops, dev, m, n, k, 730)
    res = h3synth.Bf16Array.from_f32(np.random.default_rng(731).standard_normal((m, n)).astype(np.float32))
    gate = np.random.default_rng(732).standard_normal((4, n)).astype(np.float32)
    y = ops.linear_gated_residual_mx4(am, wm, to_dev_bf16(res, dev), torch.from_numpy(gate).to(dev),
                                      to_dev_i32(cu, dev), cu)
    seg = oracle.segment_ids(cu)
    ref = oracle.gated_residual_ref(res.f32, gate, oracle.mxfp4_linear_ref(a.f32, w.f32), seg)
    terms = np.abs(oracle.mxfp4_fake_quant(a.f32)) @ np.abs(oracle.mxfp4_fake_quant(w.f32)).T
    mag = np.abs(res.f32) + np.abs(gate[seg]) * terms
    compare(to_np(y), ref, "gated residual mxfp4", mag=mag)


def test_linear_mx4_deterministic(dev, ops):
    import torch
    announce("linear mxfp4 determinism")
    a, w, am, wm = _pair(ops, dev, 700, 512, 1024, 740)
    assert torch.equal(ops.linear_mx4(am, wm), ops.linear_mx4(am, wm))


# --------------------------------------------------------------------------
# the block with MXFP4 linears
# --------------------------------------------------------------------------

def _mx4_from_storage(z):
    """What the block feeds a linear: the bf16-stored value, quantised."""
    return oracle.mxfp4_fake_quant(oracle.bf16_round(z))


def _small_inputs(lens=(300, 0, 211, 65), seed=3):
    cu = h3synth.cu_from_lengths(list(lens))
    grid = np.random.default_rng(seed).integers(0, 64, size=(int(cu[-1]), 3)).astype(np.int32)
    return h3synth.block_inputs(cu, grid, heads=4, head_dim=128, ffn=1024, seed=seed, weight_std=SMALL_STD)


def _block(ops, dev, inp, split):
    w = {nm: to_dev_bf16(getattr(inp, nm), dev) for nm in ops.WEIGHT_NAMES}
    return ops.DitBlockMX4(w, inp.heads, inp.head_dim, inp.ffn, split)


def _run(dev, blk, inp):
    cu = inp.cu_seqlens
    return blk.forward(to_dev_bf16(inp.x, dev), to_dev_bf16(inp.cond, dev), to_dev_i32(cu, dev), cu,
                       to_dev_i32(inp.grid, dev))


def _relf(a, b) -> float:
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _check_branch(x2, x, emul, emul_alt, exact, name):
    """The residual branch x2 - x against the storage-emulating MXFP4 block
    (bf16 storage at every kernel boundary, activations quantised from their
    stored values). Quantised linears turn an ulp into a whole E2M1 step, so
    the bar is calibrated on the distance between two exact emulations that
    differ only in bf16 storage: the GPU may be at most twice that far from
    the storage-emulating one, and no further from the exact block than the
    emulation plus 5e-3 (the method's quantisation floor)."""
    sens = _relf(emul_alt["x2"] - x, emul["x2"] - x)
    compare(x2 - x, emul["x2"] - x, f"{name} branch x2-x vs MXFP4 emulation",
            rel_fro=max(2.0 * sens, REL_MX_EMULATION), scaled_abs=NO_ELEMENTWISE)
    rg, re_ = _relf(x2 - x, exact["x2"] - x), _relf(emul["x2"] - x, exact["x2"] - x)
    print(f"[parity] {name}: emulation sensitivity={sens:.3e}; branch relF gpu-vs-exact={rg:.3e}, "
          f"MXFP4 emulation-vs-exact (floor)={re_:.3e}")
    assert rg <= re_ + FLOOR_MARGIN, (rg, re_)


def test_block_mx4_small(dev, ops):
    announce("block mxfp4 small (H=4, D=128, C=512, I=1024, 4 segments)")
    inp = _small_inputs()
    split = (32, 48, 48)
    out = _run(dev, _block(ops, dev, inp, split), inp)
    w = {nm: getattr(inp, nm).f32 for nm in inp.weight_names}
    args = (inp.x.f32, inp.cond.f32, w, inp.cu_seqlens, inp.grid, 4, 128, split)
    emul = oracle.dit_block_ref(*args, emulate_bf16_storage=True, linear_quant=_mx4_from_storage)
    emul_alt = oracle.dit_block_ref(*args, linear_quant=oracle.mxfp4_fake_quant)
    exact = oracle.dit_block_ref(*args)
    _check_branch(to_np(out), inp.x.f32.astype(np.float64), emul, emul_alt, exact, "small")


def test_block_mx4_zero_gates_identity_and_deterministic(dev, ops):
    announce("block mxfp4 with zero gate chunks -> x2 == x; determinism")
    inp = _small_inputs(seed=4)
    c = 512
    blk = _block(ops, dev, inp, (32, 48, 48))
    o1, o2 = bf16_bits_of(_run(dev, blk, inp)), bf16_bits_of(_run(dev, blk, inp))
    assert np.array_equal(o1, o2)
    w_mod = inp.w_mod.bits.copy()
    w_mod[2 * c:3 * c] = 0
    w_mod[5 * c:6 * c] = 0
    inp.w_mod = h3synth.Bf16Array(w_mod, h3synth.bits_to_f32(w_mod))
    out = _run(dev, _block(ops, dev, inp, (32, 48, 48)), inp)
    assert np.array_equal(bf16_bits_of(out), inp.x.bits)


def test_block_mx4_full_size_sampled_rows(dev, ops):
    """The 57,960-token block with MXFP4 linears (the launch the bench
    times): sampled tokens against the row oracle."""
    name = "block_10s_58k"
    announce(f"block mxfp4 {name} full size, sampled rows")
    wl = h3synth.WORKLOADS[name]
    inp = h3synth.workload_block_inputs(name)
    split = h3synth.rope_split_for(wl.head_dim)
    out = _run(dev, _block(ops, dev, inp, split), inp)
    n = wl.total_tokens
    rows = np.unique(np.concatenate([h3synth.sample_rows(n, 8, inp.seed), [511, 512, n - 1]]))
    rows = rows[rows < n]
    got = to_np(out[rows])
    w = {nm: getattr(inp, nm).f32 for nm in inp.weight_names}
    args = (inp.x.f32, inp.cond.f32, w, inp.cu_seqlens, inp.grid, wl.heads, wl.head_dim, split, rows)
    emul = oracle.dit_block_rows_ref(*args, emulate_bf16_storage=True, linear_quant=_mx4_from_storage)
    emul_alt = oracle.dit_block_rows_ref(*args, linear_quant=oracle.mxfp4_fake_quant)
    exact = oracle.dit_block_rows_ref(*args)
    _check_branch(got, inp.x.f32[rows].astype(np.float64), emul, emul_alt, exact, name)
