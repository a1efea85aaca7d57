"""GPU parity of the MXFP8 linears against the float64 MX emulation
(oracle.mx_linear): quantisation bit for bit, the GEMMs at the bf16 output
bar, and the SwiGLU epilogue's fused MX output within one E4M3 step (it
quantises fp32 values, the oracle float64 ones)."""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import announce, compare, to_dev_bf16, to_dev_i32, to_np, torch_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _e4m3_decode(b) -> np.ndarray:
    b = np.asarray(b).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e, m = (b >> 3) & 15, b & 7
    val = np.where(e > 0, (1.0 + m / 8.0) * np.power(2.0, e - 7), (m / 8.0) * 2.0 ** -6)
    return np.where((e == 15) & (m == 7), np.nan, sign * val)


def _scale_exponents(scales, rows, k) -> np.ndarray:
    """[rows, k/32] exponents from the K-step-major byte layout."""
    s = np.asarray(scales).astype(np.int64)
    j = np.arange(k // 32)
    r = np.arange(rows)[:, None]
    return s[((j[None, :] // 4) * rows + r) * 4 + (j[None, :] % 4)] - 127


def _mx_values(mx):
    codes = mx.codes.cpu().numpy()
    rows, k = codes.shape
    e = _scale_exponents(mx.scales.cpu().numpy(), rows, k)
    return _e4m3_decode(codes), e


def _mixed(rows, k, seed, std=1.0):
    """bf16 values with per-block magnitudes spread over 10^[-4, 4], some
    all-zero blocks, some blocks whose maximum saturates (amax just below a
    power of two times 512) and some bf16 subnormals."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)) * std
    x *= np.power(10.0, rng.uniform(-4, 4, size=(rows, k // 32))).repeat(32, axis=1)
    nb = rows * k // 32
    blocks = x.reshape(nb, 32)
    zero = rng.random(nb) < 0.05
    blocks[zero] = 0.0
    sat = rng.random(nb) < 0.05
    blocks[sat, 0] = np.sign(blocks[sat, 0] + 0.5) * 510.0 * np.power(2.0, rng.integers(-20, 20, size=sat.sum()))
    sub = rng.random(nb) < 0.02
    blocks[sub] = rng.standard_normal((sub.sum(), 32)) * 2.0 ** -130
    return h3synth.Bf16Array.from_f32(x.astype(np.float32))


@pytest.mark.parametrize("rows,k,pad", [(1, 128, 0), (37, 384, 32), (300, 640, 0)])
def test_mx_quantize_bit_exact(dev, ops, rows, k, pad):
    import torch
    announce(f"mx quantize rows={rows} k={k} row pad={pad}")
    x = _mixed(rows, k + pad, 400 + rows)
    xt = to_dev_bf16(x, dev)[:, :k]
    mx = ops.mx_quantize(xt)
    p, e = _mx_values(mx)
    pr, er = oracle.mx_quantize(x.f32.astype(np.float64)[:, :k])
    assert np.array_equal(e, er)
    assert np.array_equal(p, pr)


def _mx_pair(ops, dev, m, n, k, seed):
    a = _mixed(m, k, seed)
    w = h3synth.Bf16Array.from_f32((np.random.default_rng(seed + 1).standard_normal((n, k)) * 0.02)
                                   .astype(np.float32))
    return a, w, ops.mx_quantize(to_dev_bf16(a, dev)), ops.mx_quantize(to_dev_bf16(w, dev))


@pytest.mark.parametrize("m,n,k", [(1, 8, 128), (300, 264, 384), (513, 384, 640), (256, 256, 3072)])
def test_linear_mx_store(dev, ops, m, n, k):
    announce(f"linear mx m={m} n={n} k={k}")
    a, w, am, wm = _mx_pair(ops, dev, m, n, k, 410 + m)
    y = ops.linear_mx(am, wm)
    ref = oracle.mx_linear_ref(a.f32, w.f32)
    # block magnitudes span 10^[-4, 4]: an output's rounding error scales
    # with the sum of its terms' magnitudes, not with its (cancelled) value
    mag = np.abs(oracle.mx_fake_quant(a.f32)) @ np.abs(oracle.mx_fake_quant(w.f32)).T
    compare(to_np(y), ref, f"linear mx m={m} n={n} k={k}", mag=mag)


@pytest.mark.parametrize("m,n,k", [(333, 256, 384), (600, 128, 640)])
def test_linear_swiglu_mx(dev, ops, m, n, k):
    announce(f"linear swiglu mx m={m} n={n} k={k}")
    rng = np.random.default_rng(420 + m)
    a = h3synth.Bf16Array.from_f32(rng.standard_normal((m, k)).astype(np.float32))
    wg = h3synth.Bf16Array.from_f32((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    wu = h3synth.Bf16Array.from_f32((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    q = lambda t: ops.mx_quantize(to_dev_bf16(t, dev))
    y = ops.linear_swiglu_mx(q(a), q(wg), q(wu))
    p, e = _mx_values(y)
    got = p * np.power(2.0, e.astype(np.float64)).repeat(32, axis=1)
    fq = oracle.mx_fake_quant
    aq, gq, uq = fq(a.f32), fq(wg.f32), fq(wu.f32)
    pre = oracle.swiglu_ref(aq, gq, uq)
    pr, er = oracle.mx_quantize(pre)
    ref = oracle.mx_dequantize(pr, er)
    # The kernel quantises its fp32 product; the matrix core's accumulation
    # error is measured at ~2^-19 of the sum of the terms' magnitudes (it
    # shows where g or u cancels to ~1e-5 of its terms), so allow eps = 2^-16
    # of that, propagated through silu(g) u, plus half an E4M3 step at the
    # block's scale; where fp32 and float64 straddle a power of two the
    # block exponent may be one off.
    assert np.mean(e != er) < 1e-3 and np.all(np.abs(e - er) <= 1)
    eps = 2.0 ** -16
    g, u = aq @ gq.T, aq @ uq.T
    tg, tu = np.abs(aq) @ np.abs(gq).T, np.abs(aq) @ np.abs(uq).T
    d_pre = 1.1 * eps * tg * np.abs(u) + np.abs(oracle.silu(g)) * eps * tu + eps * np.abs(pre)
    scale = np.power(2.0, e.astype(np.float64)).repeat(32, axis=1)
    v = np.abs(pre) / scale
    half = 0.5 * np.power(2.0, np.maximum(np.floor(np.log2(np.maximum(v, 2.0 ** -30))), -6) - 3) * scale
    over = np.abs(got - pre) - (d_pre + half * (1 + 1e-9))
    sat = v > 448
    assert np.all(over[~sat] <= 0), float(over[~sat].max())
    assert np.all(np.abs(got[sat]) == 448 * scale[sat])          # saturated codes
    assert np.mean(got == ref) > 0.99
    compare(got, pre, "swiglu mx vs unquantised product", rel_fro=5e-2, scaled_abs=0.5)


def test_linear_gated_residual_mx_multi_segment(dev, ops):
    import torch
    announce("linear gated residual mx, 3 segments")
    lens = [100, 0, 157, 300]
    cu = h3synth.cu_from_lengths(lens)
    m, n, k = int(cu[-1]), 392, 384
    a, w, am, wm = _mx_pair(ops, dev, m, n, k, 430)
    res = h3synth.Bf16Array.from_f32(np.random.default_rng(431).standard_normal((m, n)).astype(np.float32))
    gate = np.random.default_rng(432).standard_normal((4, n)).astype(np.float32)
    y = ops.linear_gated_residual_mx(am, wm, to_dev_bf16(res, dev), torch.from_numpy(gate).to(dev),
                                     to_dev_i32(cu, dev), cu)
    seg = oracle.segment_ids(cu)
    ref = oracle.gated_residual_ref(res.f32, gate, oracle.mx_linear_ref(a.f32, w.f32), seg)
    terms = np.abs(oracle.mx_fake_quant(a.f32)) @ np.abs(oracle.mx_fake_quant(w.f32)).T
    mag = np.abs(res.f32) + np.abs(gate[seg]) * terms
    compare(to_np(y), ref, "gated residual mx", mag=mag)


def test_linear_mx_deterministic(dev, ops):
    import torch
    announce("linear mx determinism")
    a, w, am, wm = _mx_pair(ops, dev, 700, 512, 1024, 440)
    y1 = ops.linear_mx(am, wm)
    y2 = ops.linear_mx(am, wm)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("c", [512, 3072])
def test_adaln_mx_multi_segment(dev, ops, c):
    """AdaLN with MX output against MX(the float64 AdaLN): the kernel
    quantises its fp32 values, so a code may sit one E4M3 step off where the
    value is within fp32 rounding (2^-18 relative, generous) of a midpoint."""
    import torch
    announce(f"adaln mx C={c}")
    lens = [300, 0, 65, 129]
    cu = h3synth.cu_from_lengths(lens)
    n = int(cu[-1])
    rng = np.random.default_rng(450 + c)
    x = h3synth.Bf16Array.from_f32(rng.standard_normal((n, c)).astype(np.float32))
    mod = (rng.standard_normal((len(lens), 6 * c)) * 0.5).astype(np.float32)
    mod_t = torch.from_numpy(mod).to(dev)
    h = ops.adaln_rmsnorm_modulate_mx(to_dev_bf16(x, dev), mod_t[:, 0:c], mod_t[:, c:2 * c],
                                      to_dev_i32(cu, dev), cu, 1e-6)
    p, e = _mx_values(h)
    seg = oracle.segment_ids(cu)
    pre = oracle.adaln_modulate_ref(x.f32, mod[:, 0:c], mod[:, c:2 * c], seg, 1e-6)
    pr, er = oracle.mx_quantize(pre)
    assert np.mean(e != er) < 1e-3 and np.all(np.abs(e - er) <= 1)
    scale = np.power(2.0, e.astype(np.float64)).repeat(32, axis=1)
    got = p * scale
    v = np.abs(pre) / scale
    half = 0.5 * np.power(2.0, np.maximum(np.floor(np.log2(np.maximum(v, 2.0 ** -30))), -6) - 3) * scale
    sat = v > 448
    over = np.abs(got - pre) - (half * (1 + 1e-9) + 2.0 ** -18 * np.abs(pre))
    assert np.all(over[~sat] <= 0), float(over[~sat].max())
    assert np.all(np.abs(got[sat]) == 448 * scale[sat])
    assert np.mean(got == oracle.mx_dequantize(pr, er)) > 0.999
