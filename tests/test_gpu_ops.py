"""GPU parity of the per-block fused operators: Q/K RMSNorm + 3D RoPE,
AdaLN modulation + RMSNorm, and the MFMA GEMMs with their epilogues."""
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


def _bf(shape, seed, std=1.0, mean=0.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std) + np.float32(mean)
    return h3synth.Bf16Array.from_f32(a)


def test_qk_norm_rope_video_grid_d128(dev, ops):
    """head_dim 128, split 32/48/48, positions of a real packed request
    (text + audio + 3 video frames of 24 x 42)."""
    announce("qk norm+rope D=128 on a packed text/audio/video request")
    req = h3synth.Request(512, 1000, 3)
    cu, grid = h3synth.pack([req])
    inp = h3synth.attention_inputs(cu, grid, 6, 128, seed=21)
    q, k = to_dev_bf16(inp.q, dev), to_dev_bf16(inp.k, dev)
    split = h3synth.rope_split_for(128)
    ops.qk_rmsnorm_rope(q, k, to_dev_bf16(inp.w_q, dev), to_dev_bf16(inp.w_k, dev),
                        to_dev_i32(grid, dev), split, 1e4, 1e-6)
    qr, kr = oracle.qk_norm_rope_ref(inp.q.f32, inp.k.f32, inp.w_q.f32, inp.w_k.f32, grid,
                                     split, 1e4, 1e-6)
    compare(to_np(q), qr, "q norm+rope D128")
    compare(to_np(k), kr, "k norm+rope D128")


def test_qk_norm_rope_in_place_on_packed_qkv(dev, ops):
    import torch
    announce("qk norm+rope strided in a qkv buffer, v untouched")
    n, heads, d = 333, 4, 128
    qkv = _bf((n, 3 * heads * d), 22)
    grid = np.random.default_rng(23).integers(0, 1500, size=(n, 3)).astype(np.int32)
    wq, wk = _bf((d,), 24, 0.1, 1.0), _bf((d,), 25, 0.1, 1.0)
    t = to_dev_bf16(qkv, dev)
    before_v = t[:, 2 * heads * d:].clone()
    c = heads * d
    ops.qk_rmsnorm_rope(t[:, :c].view(n, heads, d), t[:, c:2 * c].view(n, heads, d),
                        to_dev_bf16(wq, dev), to_dev_bf16(wk, dev), to_dev_i32(grid, dev),
                        (32, 48, 48), 1e4, 1e-6)
    q = qkv.f32[:, :c].reshape(n, heads, d)
    k = qkv.f32[:, c:2 * c].reshape(n, heads, d)
    qr, kr = oracle.qk_norm_rope_ref(q, k, wq.f32, wk.f32, grid, (32, 48, 48), 1e4, 1e-6)
    compare(to_np(t[:, :c]).reshape(n, heads, d), qr, "q strided")
    compare(to_np(t[:, c:2 * c]).reshape(n, heads, d), kr, "k strided")
    assert torch.equal(t[:, 2 * c:], before_v)


@pytest.mark.parametrize("b", [1, 3, 6])
def test_modulation(dev, ops, b):
    """B = 6 spans two passes of the kernel's staged segment chunk."""
    announce(f"modulation GEMV B={b} C=3072")
    c = 3072
    cond = _bf((b, c), 30)
    w = _bf((6 * c, c), 31, 0.02)
    mod = ops.modulation(to_dev_bf16(cond, dev), to_dev_bf16(w, dev))
    ref = oracle.modulation_ref(cond.f32, w.f32)
    compare(to_np(mod), ref, "modulation", rel_fro=1e-5, scaled_abs=1e-5)


@pytest.mark.parametrize("c", [512, 3072])
def test_adaln_multi_segment(dev, ops, c):
    announce(f"adaln rmsnorm+modulate C={c}, 4 segments")
    lens = [7, 0, 300, 45]
    cu = h3synth.cu_from_lengths(lens)
    n = int(cu[-1])
    x = _bf((n, c), 40)
    mod = np.random.default_rng(41).standard_normal((len(lens), 6 * c)).astype(np.float32)
    import torch
    mod_t = torch.from_numpy(mod).to(dev)
    h = ops.adaln_rmsnorm_modulate(to_dev_bf16(x, dev), mod_t[:, 0:c], mod_t[:, c:2 * c],
                                   to_dev_i32(cu, dev), cu, 1e-6)
    seg = oracle.segment_ids(cu)
    ref = oracle.adaln_modulate_ref(x.f32, mod[:, 0:c], mod[:, c:2 * c], seg, 1e-6)
    compare(to_np(h), ref, f"adaln C={c}")


@pytest.mark.parametrize("m,n", [(1, 384), (300, 384), (1000, 384), (513, 264), (257, 8)])
def test_linear_store(dev, ops, m, n):
    """Ragged in both tile dimensions (256 x 256 tiles)."""
    announce(f"linear store m={m} n={n}")
    k = 512
    a, w = _bf((m, k), 50), _bf((n, k), 51, 0.05)
    y = ops.linear(to_dev_bf16(a, dev), to_dev_bf16(w, dev))
    compare(to_np(y), a.f32.astype(np.float64) @ w.f32.astype(np.float64).T, f"linear m={m} n={n}")


@pytest.mark.parametrize("m,n", [(333, 256), (600, 200)])
def test_linear_swiglu(dev, ops, m, n):
    announce(f"linear swiglu m={m} n={n}")
    k = 640
    a = _bf((m, k), 52)
    wg, wu = _bf((n, k), 53, 0.05), _bf((n, k), 54, 0.05)
    y = ops.linear_swiglu(to_dev_bf16(a, dev), to_dev_bf16(wg, dev), to_dev_bf16(wu, dev))
    compare(to_np(y), oracle.swiglu_ref(a.f32, wg.f32, wu.f32), "swiglu")


def test_linear_gated_residual_multi_segment(dev, ops):
    import torch
    announce("linear gated residual, 3 segments")
    lens = [100, 0, 157, 300]
    cu = h3synth.cu_from_lengths(lens)
    m, n, k = int(cu[-1]), 392, 384
    a, w, res = _bf((m, k), 55), _bf((n, k), 56, 0.05), _bf((m, n), 57)
    gate = np.random.default_rng(58).standard_normal((4, 6 * n)).astype(np.float32)
    gate_t = torch.from_numpy(gate).to(dev)
    y = ops.linear_gated_residual(to_dev_bf16(a, dev), to_dev_bf16(w, dev), to_dev_bf16(res, dev),
                                  gate_t[:, 2 * n:3 * n], to_dev_i32(cu, dev), cu)
    seg = oracle.segment_ids(cu)
    ref = oracle.gated_residual_ref(res.f32, gate[:, 2 * n:3 * n], a.f32.astype(np.float64)
                                    @ w.f32.astype(np.float64).T, seg)
    compare(to_np(y), ref, "gated residual")


def test_gated_residual_in_place(dev, ops):
    """y may alias res: each element is read before it is written."""
    import torch
    announce("gated residual in place")
    cu = h3synth.cu_from_lengths([130])
    m, n, k = 130, 128, 64
    a, w, res = _bf((m, k), 60), _bf((n, k), 61, 0.05), _bf((m, n), 62)
    gate = torch.ones((1, n), dtype=torch.float32, device=dev)
    r = to_dev_bf16(res, dev)
    ops.linear_gated_residual(to_dev_bf16(a, dev), to_dev_bf16(w, dev), r, gate,
                              to_dev_i32(cu, dev), cu, out=r)
    ref = res.f32 + a.f32.astype(np.float64) @ w.f32.astype(np.float64).T
    compare(to_np(r), ref, "gated residual in place")


def test_gated_residual_8_byte_aligned_views(dev, ops):
    """res and y 8-byte but not 16-byte aligned (the epilogue's 8-byte path),
    ragged in both tile dimensions."""
    import torch
    announce("gated residual, 8-byte aligned res / y views")
    cu = h3synth.cu_from_lengths([170, 131])
    m, n, k = 301, 264, 128
    a, w, res = _bf((m, k), 63), _bf((n, k), 64, 0.05), _bf((m, n), 65)
    gate = np.random.default_rng(66).standard_normal((2, n)).astype(np.float32)
    r_big = torch.zeros(m * n + 4, dtype=torch.bfloat16, device=dev)
    r = r_big[4:].view(m, n)
    r.copy_(to_dev_bf16(res, dev))
    y_big = torch.zeros(m * n + 4, dtype=torch.bfloat16, device=dev)
    y = y_big[4:].view(m, n)
    assert r.data_ptr() % 16 == 8 and y.data_ptr() % 16 == 8
    ops.linear_gated_residual(to_dev_bf16(a, dev), to_dev_bf16(w, dev), r,
                              torch.from_numpy(gate).to(dev), to_dev_i32(cu, dev), cu, out=y)
    seg = oracle.segment_ids(cu)
    ref = oracle.gated_residual_ref(res.f32, gate, a.f32.astype(np.float64)
                                    @ w.f32.astype(np.float64).T, seg)
    compare(to_np(y), ref, "gated residual 8-byte views")
    assert float(y_big[:4].float().abs().sum()) == 0.0      # nothing written before y
