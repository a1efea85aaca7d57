"""GPU parity of the fp8 path: e4m3 quantisation (codes and scales bit-exact
against the oracle) and fp8 attention with skip-softmax (against the float64
fp8 emulation at the 1e-2 bar, and against exact attention).

Against exact attention the quantisation itself sets a floor: the float64
emulation of the same fp8 scheme is already about 5e-2 (relative Frobenius)
away from exact attention on i.i.d. N(0,1) inputs, so the kernel is required
to add no more than 5e-3 on top of that floor, and the literal 5e-2 outcome
is printed beside it."""
import numpy as np
import pytest

import h3synth
import oracle
from _gpu_helpers import announce, compare, to_dev_bf16, to_dev_i32, to_np, torch_device

pytestmark = pytest.mark.gpu

REL_FP8_EXACT = 5e-2     # fp8 path against exact attention (relative Frobenius), reported
FLOOR_MARGIN = 5e-3      # allowed excess of the kernel over the emulated fp8 floor
# Elementwise bar of the fp8 path against its emulation: the fp8 bar, 5e-2 of
# max(1, |ref|). The kernel sums the encoded P for the softmax denominator
# while the emulation sums the unquantised p; on peaked rows that moves single
# outputs by up to about 2 % (relative Frobenius error stays near 3e-3, held
# to 1e-2).
SCALED_ABS_FP8 = 5e-2
D = 128


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _e4m3_decode(b) -> np.ndarray:
    """OCP e4m3fn byte -> value (bias 7, subnormals 2^-6 * m/8, 0x7f/0xff NaN)."""
    b = np.asarray(b).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e, m = (b >> 3) & 15, b & 7
    val = np.where(e > 0, (1.0 + m / 8.0) * np.power(2.0, e - 7), (m / 8.0) * 2.0 ** -6)
    return np.where((e == 15) & (m == 7), np.nan, sign * val)


def _tile_position() -> np.ndarray:
    """Position of key j (0..63) inside a v8t tile row (the layout in h3dit.h)."""
    pos = np.zeros(64, dtype=np.int64)
    for j in range(64):
        b, r = j >> 5, j & 31
        pos[j] = 32 * ((r >> 2) & 1) + 16 * b + 4 * (r >> 3) + (r & 3)
    return pos


def _scaled_inputs(lens, heads, seed):
    """bf16 q, k, v [N, H, 128] with per-token magnitudes spread over 10^[-2, 2]
    so that block and channel scales differ widely."""
    cu = h3synth.cu_from_lengths(lens)
    n = int(cu[-1])
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        a = rng.standard_normal((n, heads, D)).astype(np.float32)
        a *= np.power(10.0, rng.uniform(-2, 2, size=(n, 1, 1))).astype(np.float32)
        out.append(h3synth.Bf16Array.from_f32(a))
    return cu, out


def _assert_quantize_matches(ops, res, q, k, v, cu, lens, heads):
    """Codes and scales of h3_fp8_quantize equal the oracle's bit for bit."""
    qc, qs = oracle.quantize_qk_blocks(q.f32, cu, 64)
    kc, ks = oracle.quantize_qk_blocks(k.f32, cu, 64)
    vc, vs = oracle.quantize_v_channels(v.f32, cu)
    assert np.array_equal(res["q_scale"].cpu().numpy(), qs.astype(np.float32))
    assert np.array_equal(res["k_scale"].cpu().numpy(), ks.astype(np.float32))
    assert np.array_equal(res["v_scale"].cpu().numpy(), vs.astype(np.float32))
    assert np.array_equal(_e4m3_decode(res["q8"].cpu().numpy()), qc)
    k8 = _e4m3_decode(res["k8"].cpu().numpy())     # [H, T, 64, 128]
    v8 = _e4m3_decode(res["v8t"].cpu().numpy())    # [H, T, 128, 64]
    pos = _tile_position()
    tile = 0
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        for t0 in range(a, b, 64):
            rows = min(64, b - t0)
            want_k = np.zeros((heads, 64, D))
            want_k[:, :rows] = kc[t0:t0 + rows].transpose(1, 0, 2)
            assert np.array_equal(k8[:, tile], want_k), (s, t0)
            want_v = np.zeros((heads, D, 64))
            want_v[:, :, pos[:rows]] = vc[t0:t0 + rows].transpose(1, 2, 0)
            assert np.array_equal(v8[:, tile], want_v), (s, t0)
            tile += 1
    assert tile == k8.shape[1] == ops.fp8_num_tiles(cu)


@pytest.mark.parametrize("lens", [[100, 0, 64, 257, 1], [65], [0, 3, 0]])
def test_fp8_quantize_codes_and_scales_bit_exact(dev, ops, lens):
    heads = 3
    announce(f"fp8 quantise lens={lens} H={heads}")
    cu, (q, k, v) = _scaled_inputs(lens, heads, 301)
    res = ops.fp8_quantize(to_dev_bf16(q, dev), to_dev_bf16(k, dev), to_dev_bf16(v, dev),
                           to_dev_i32(cu, dev), cu)
    _assert_quantize_matches(ops, res, q, k, v, cu, lens, heads)


def _e4m3_midpoints() -> np.ndarray:
    vals = [m * 2.0 ** -9 for m in range(8)]
    vals += [(1 + m / 8) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
    grid = np.array([x for x in vals if x <= 448.0])
    return (grid[:-1] + grid[1:]) / 2


def _pattern(kind, rows, rng) -> np.ndarray:
    """[rows, 128] float32 values that are exact bf16 numbers.
    ties(a): +-m a / 448 for e4m3 midpoints m, with one +-a in every column, so
    every block and channel has amax a and many quotients 448 x / a are exact
    midpoints; 24.5 makes 448 / a inexact in fp32, 24.5 * 2^-70 takes the
    pre-scaled path for tiny blocks. subnormal: bf16 subnormals only."""
    tie_amax = {"ties448": 448.0, "ties24": 24.5, "tiny": 24.5 * 2.0 ** -70}
    if kind in tie_amax:
        amax = tie_amax[kind]
        x = rng.choice(_e4m3_midpoints(), size=(rows, D)) * amax / 448.0
        x[rng.integers(0, rows, size=D), np.arange(D)] = amax
        x *= rng.choice([-1.0, 1.0], size=(rows, D))
        return x.astype(np.float32)
    if kind == "subnormal":
        bits = (rng.integers(1, 128, size=(rows, D)).astype(np.uint32) << 16)
        bits |= rng.integers(0, 2, size=(rows, D)).astype(np.uint32) << 31
        return bits.view(np.float32)
    if kind == "zero":
        return np.zeros((rows, D), np.float32)
    x = rng.standard_normal((rows, D)) * np.power(10.0, rng.uniform(-2, 2, size=(rows, 1)))
    return h3synth.Bf16Array.from_f32(x.astype(np.float32)).f32


def test_fp8_quantize_ties_tiny_subnormal_and_zero_blocks(dev, ops):
    """Blocks and channels built so that the code decision meets its edge
    cases: exact rounding midpoints (ties to even) with exact and inexact
    448 / amax, blocks with amax below 2^-64, bf16 subnormals, all-zero
    blocks and channels, and a ragged last tile."""
    lens = [64, 64, 64, 100, 1]
    heads = 2
    kinds = [("ties448", "ties24"), ("tiny", "subnormal"), ("zero", "random"),
             ("random", "random"), ("random", "ties24")]
    announce(f"fp8 quantise edge blocks lens={lens} H={heads}")
    cu = h3synth.cu_from_lengths(lens)
    n = int(cu[-1])
    rng = np.random.default_rng(303)
    arrays = []
    for t in range(3):
        a = np.zeros((n, heads, D), np.float32)
        for s, (k0, k1) in enumerate(kinds):
            r0, r1 = int(cu[s]), int(cu[s + 1])
            a[r0:r1, 0] = _pattern(k0, r1 - r0, rng)
            a[r0:r1, 1] = _pattern(k1, r1 - r0, rng)
        if t == 2:
            a[int(cu[3]):int(cu[4]), 0, 5:9] = 0.0          # zero V channels in one segment
        b = h3synth.Bf16Array.from_f32(a)
        assert np.array_equal(b.f32, a)                     # every value is a bf16 number
        arrays.append(b)
    q, k, v = arrays
    res = ops.fp8_quantize(to_dev_bf16(q, dev), to_dev_bf16(k, dev), to_dev_bf16(v, dev),
                           to_dev_i32(cu, dev), cu)
    _assert_quantize_matches(ops, res, q, k, v, cu, lens, heads)


def _relf(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _check_vs_exact(got, emu, exact, name):
    """The kernel's distance to exact attention may exceed the emulated fp8
    floor by at most FLOOR_MARGIN; the literal 5e-2 bar is reported."""
    rg, re_ = _relf(got, exact), _relf(emu, exact)
    print(f"[parity] {name}: relF gpu-vs-exact={rg:.3e} emulation-vs-exact (fp8 floor)={re_:.3e} "
          f"literal 5e-2 bar {'met' if rg <= REL_FP8_EXACT else 'not met (floor)'}")
    assert np.all(np.isfinite(got))
    assert rg <= re_ + FLOOR_MARGIN, (rg, re_)


def _fp8_attn(ops, dev, q, k, v, cu, skip=False, thr=8.0):
    import torch
    n_items = ops.attn_num_items(cu, q.shape[1])
    counts = torch.full((max(n_items, 1),), -1, dtype=torch.int32, device=dev)
    out = ops.attn_varlen(to_dev_bf16(q, dev), to_dev_bf16(k, dev), to_dev_bf16(v, dev),
                          to_dev_i32(cu, dev), cu, precision="fp8", skip_softmax=skip,
                          skip_threshold=thr, skip_counts=counts)
    return out, counts[:n_items].cpu().numpy()


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 0, 300, 700], [2000]])
def test_fp8_attention_matches_emulation_and_exact(dev, ops, lens):
    heads = 2
    announce(f"fp8 attention lens={lens} H={heads}")
    cu = h3synth.cu_from_lengths(lens)
    grid = np.zeros((int(cu[-1]), 3), np.int32)
    inp = h3synth.attention_inputs(cu, grid, heads, D, seed=311)
    out, counts = _fp8_attn(ops, dev, inp.q, inp.k, inp.v, cu)
    emu, _ = oracle.fp8_attn_emulated_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    exact = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    got = to_np(out)
    compare(got, emu, f"fp8 vs fp8 emulation lens={lens}", scaled_abs=SCALED_ABS_FP8)
    _check_vs_exact(got, emu, exact, f"fp8 vs exact lens={lens}")
    assert (counts == 0).all()


def test_fp8_skip_softmax_frame_local(dev, ops):
    """Frame-local inputs (keys of a query's own 1008-token frame gain ~12 in
    the logit) make most key tiles skippable; the skipped fraction must match
    the emulation within 0.5 % absolute, the output the emulation's bar."""
    heads = 2
    reqs = [h3synth.Request(64, 128, 3), h3synth.Request(32, 96, 4)]
    cu, _ = h3synth.pack(reqs)
    announce(f"fp8 skip-softmax frame-local cu={cu.tolist()} H={heads}")
    inp = h3synth.frame_local_attention_inputs(cu, heads, D, seed=321)
    out, counts = _fp8_attn(ops, dev, inp.q, inp.k, inp.v, cu, skip=True)
    emu, report = oracle.fp8_attn_emulated_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu, skip=True,
                                               threshold=8.0)
    skipped = sum(r[2] for r in report)
    pairs = sum(r[3] for r in report)
    frac_emu = skipped / pairs
    frac_gpu = counts.sum() / pairs
    print(f"[parity] skip fraction gpu={frac_gpu:.4f} emulation={frac_emu:.4f} pairs={pairs}")
    assert frac_emu > 0.3, "the case must exercise skipping"
    assert abs(frac_gpu - frac_emu) <= 0.005
    got = to_np(out)
    compare(got, emu, "fp8+skip vs emulation", scaled_abs=SCALED_ABS_FP8)
    exact = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
    _check_vs_exact(got, emu, exact, "fp8+skip vs exact")


def test_fp8_skip_counts_per_item_and_determinism(dev, ops):
    """Per-item counts equal the emulation's per-group counts summed over the
    item's eight 32-row groups, up to borderline tiles; two runs are bitwise
    identical."""
    import torch
    heads = 2
    cu, _ = h3synth.pack([h3synth.Request(64, 128, 3)])
    inp = h3synth.frame_local_attention_inputs(cu, heads, D, seed=331)
    o1, c1 = _fp8_attn(ops, dev, inp.q, inp.k, inp.v, cu, skip=True)
    o2, c2 = _fp8_attn(ops, dev, inp.q, inp.k, inp.v, cu, skip=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert np.array_equal(c1, c2)
    _, report = oracle.fp8_attn_emulated_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu, skip=True)
    items = ops.build_schedule_host(cu, heads)
    per_group = {(h, t0): ns for h, t0, ns, _ in report}
    diffs = []
    for i, (h, s, q0, qlen) in enumerate(items):
        want = sum(per_group[(h, t)] for t in range(q0, q0 + qlen, 32))
        diffs.append(abs(int(c1[i]) - want))
    total = sum(r[3] for r in report)
    assert sum(diffs) <= 0.005 * total, (sum(diffs), total)


def test_fp8_full_size_sampled_groups(dev, ops):
    """58k tokens, 24 heads: the whole fp8 pass on the GPU (the configuration
    the bench times), 10 sampled 32-row groups against the emulation and the
    exact attention, on two heads (quantisation is per head)."""
    w = h3synth.WORKLOADS["attn_fp8_10s_58k"]
    inp = h3synth.workload_attention_inputs(w.name)
    cu = inp.cu_seqlens
    n = int(cu[-1])
    announce(f"fp8 full size N={n} H={w.heads} sampled groups")
    out, _ = _fp8_attn(ops, dev, inp.q, inp.k, inp.v, cu, skip=True)
    hs = [3, 17]
    rng = np.random.default_rng(341)
    starts = sorted({0, 32 * ((n - 1) // 32)} | set((32 * rng.integers(0, n // 32, 8)).tolist()))
    groups = [(i % 2, t0) for i, t0 in enumerate(starts)]
    q, k, v = (a.f32[:, hs] for a in (inp.q, inp.k, inp.v))
    emu, _ = oracle.fp8_attn_emulated_ref(q, k, v, cu, skip=True, groups=groups)
    rows = np.array(sorted({t for _, t0 in groups for t in range(t0, min(n, t0 + 32))}))
    import torch
    got_all = to_np(out.index_select(0, torch.from_numpy(rows).to(dev))[:, hs])
    sel_emu = np.zeros_like(got_all)
    sel_got = np.zeros_like(got_all)
    row_idx = {t: i for i, t in enumerate(rows)}
    for hi, t0 in groups:
        for t in range(t0, min(n, t0 + 32)):
            sel_emu[row_idx[t], hi] = emu[t, hi]
            sel_got[row_idx[t], hi] = got_all[row_idx[t], hi]
    compare(sel_got, sel_emu, "fp8 58k sampled vs emulation", scaled_abs=SCALED_ABS_FP8)
    exact = oracle.attn_varlen_ref(q, k, v, cu, rows=rows)
    mask = np.zeros_like(got_all, dtype=bool)
    for hi, t0 in groups:
        for t in range(t0, min(n, t0 + 32)):
            mask[row_idx[t], hi] = True
    _check_vs_exact(np.where(mask, got_all, 0), np.where(mask, sel_emu, 0) + 0.0,
                    np.where(mask, exact, 0), "fp8 58k sampled vs exact")


@pytest.mark.xfail(strict=True, raises=AssertionError,
                   reason="the literal 5e-2 relative bar against float64 attention is not met at "
                          "this shape: the e4m3 quantisation of Q, K, P and V itself (the float64 "
                          "emulation) is 5.1-5.6e-2 from exact attention on i.i.d. inputs")
def test_fp8_c4_literal_bar_against_exact(dev, ops):
    """The 58k-token, 24 x 128 fp8 attention (skip on) against exact float64
    attention on 16 sampled 32-row groups of two heads, held to the literal
    5e-2 relative Frobenius bar. Expected to fail (strict): the method's own
    quantisation floor lies above the bar; the margin over that floor is
    checked by test_fp8_full_size_sampled_groups."""
    import torch
    w = h3synth.WORKLOADS["attn_fp8_10s_58k"]
    inp = h3synth.workload_attention_inputs(w.name)
    cu = inp.cu_seqlens
    n = int(cu[-1])
    announce(f"fp8 C4 literal 5e-2 bar N={n} H={w.heads}")
    out, _ = _fp8_attn(ops, dev, inp.q, inp.k, inp.v, cu, skip=True)
    hs = [1, 11]
    rng = np.random.default_rng(351)
    starts = sorted(set((32 * rng.integers(0, n // 32, 16)).tolist()))
    rows = np.array(sorted({t for t0 in starts for t in range(t0, min(n, t0 + 32))}))
    got = to_np(out.index_select(0, torch.from_numpy(rows).to(dev))[:, hs])
    exact = oracle.attn_varlen_ref(inp.q.f32[:, hs], inp.k.f32[:, hs], inp.v.f32[:, hs], cu, rows=rows)
    rg = _relf(got, exact)
    print(f"[parity] fp8 C4 sampled rows vs exact: relF={rg:.3e} (literal bar {REL_FP8_EXACT})")
    assert rg <= REL_FP8_EXACT, f"relF {rg:.3e} > {REL_FP8_EXACT}"
