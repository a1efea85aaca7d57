"""Pins of the fp8 (e4m3) emulation: the format grid, block scaling, the
tiled online softmax and the skip rule (CPU only)."""
import math
import os

import numpy as np
import pytest

from oracle import attn_varlen_ref, e4m3_round, fp8_attn_emulated_ref
from oracle import quantize_qk_blocks, quantize_v_channels

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def _rand(shape, seed, std=1.0):
    return std * np.random.default_rng(seed).standard_normal(shape)


def _positive_e4m3_grid():
    vals = [m * 2.0 ** -9 for m in range(1, 8)]                     # subnormals
    for e in range(-6, 9):
        for m in range(8):
            vals.append((1 + m / 8) * 2.0 ** e)
    return np.array([v for v in vals if v <= 448.0])


def test_grid_points_are_fixed_points():
    g = _positive_e4m3_grid()
    assert g.size == 126 and g.max() == 448.0 and g.min() == 2.0 ** -9
    assert np.array_equal(e4m3_round(g), g)
    assert np.array_equal(e4m3_round(-g), -g)


def test_golden_rounding_table():
    """Rounding cases from the OCP 8-bit floating point specification's
    E4M3 definition (max normal 448, min subnormal 2^-9, ties to even)."""
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                rows.append((float.fromhex(a) if a.startswith(("0x", "-0x")) else float(a),
                             float.fromhex(b) if b.startswith(("0x", "-0x")) else float(b)))
    assert len(rows) >= 10
    for a, b in rows:
        assert e4m3_round(a) == b, (a, b)


def test_matches_torch_float8_cast_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000),
                        rng.standard_normal(20000) * 1e-2, rng.standard_normal(5000) * 1e-3])
    a = a.astype(np.float32).astype(np.float64)      # torch casts from float32
    t = torch.from_numpy(a.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64)
    assert np.array_equal(e4m3_round(a), t.numpy())


def test_block_quantisation_is_segment_aligned():
    cu = [0, 5, 75]
    n, heads, d = 75, 2, 8
    x = _rand((n, heads, d), 4)
    x[68, 1, 3] = 1000.0          # in the first block of segment 1 ([5, 69))
    codes, scales = quantize_qk_blocks(x, cu, 64)
    assert scales.shape == (3, heads)               # [0,5), [5,69), [69,75)
    assert scales[1, 1] == pytest.approx(1000.0 / 448.0)
    assert scales[2, 1] == pytest.approx(np.abs(x[69:75, 1]).max() / 448.0)
    # values on the grid with amax exactly 448 are reproduced, scale 1
    y = np.sign(_rand((64, 1, 4), 5)) * _positive_e4m3_grid()[np.random.default_rng(6)
                                                               .integers(0, 126, (64, 1, 4))]
    y[0, 0, 0] = 448.0
    c2, s2 = quantize_qk_blocks(y, [0, 64], 64)
    assert np.array_equal(c2, y) and s2.tolist() == [[1.0]]
    zc, zs = quantize_qk_blocks(np.zeros((3, 1, 4)), [0, 3], 64)
    assert zs.tolist() == [[1.0]] and not zc.any()


def test_v_channel_scales():
    cu = [0, 10, 30]
    v = _rand((30, 2, 4), 7)
    codes, scales = quantize_v_channels(v, cu)
    assert scales.shape == (2, 2, 4)
    assert scales[1, 0, 2] == pytest.approx(np.abs(v[10:30, 0, 2]).max() / 448.0)
    assert np.max(np.abs(codes)) <= 448.0


def test_unquantised_tiled_online_softmax_equals_exact():
    cu = [0, 1, 130, 130, 400]
    q, k, v = _rand((400, 2, 16), 8, 2.0), _rand((400, 2, 16), 9, 2.0), _rand((400, 2, 16), 10)
    out, rep = fp8_attn_emulated_ref(q, k, v, cu, quantize=False)
    ref = attn_varlen_ref(q, k, v, cu)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert all(r[2] == 0 for r in rep)


def test_quantised_error_is_near_the_fp8_floor():
    # i.i.d. N(0,1), D = 128, one segment: the error of e4m3 Q/K/P/V relative
    # to the exact result sits around 5e-2 (three 4-bit-mantissa roundings)
    cu = [0, 1024]
    q, k, v = _rand((1024, 1, 128), 11), _rand((1024, 1, 128), 12), _rand((1024, 1, 128), 13)
    out, _ = fp8_attn_emulated_ref(q, k, v, cu)
    ref = attn_varlen_ref(q, k, v, cu)
    err = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 0.02 < err < 0.08


def test_skip_rule():
    d = 16
    n = 256
    k = _rand((n, 1, d), 14, 0.1)
    q = np.repeat(_rand((1, 1, d), 15), n, axis=0)
    v = _rand((n, 1, d), 16)
    k[3] = 40.0 * q[0] / np.linalg.norm(q[0])      # one dominating key in tile 0
    cu = [0, n]
    base, rep0 = fp8_attn_emulated_ref(q, k, v, cu, quantize=False, skip=False)
    out, rep = fp8_attn_emulated_ref(q, k, v, cu, quantize=False, skip=True, threshold=8.0)
    assert all(r[2] == 0 for r in rep0)
    # every later tile of every 32-row group is far below the running max
    assert all(r[2] == r[3] - 1 for r in rep) and rep[0][3] == 4
    # a skipped tile only drops terms below exp(-8) relative to the max term
    assert np.max(np.abs(out - base)) < 64 * 3 * math.exp(-8) * np.abs(v).max()
    # an infinite threshold never skips and changes nothing
    out2, rep2 = fp8_attn_emulated_ref(q, k, v, cu, quantize=False, skip=True,
                                       threshold=np.inf)
    assert np.array_equal(out2, base) and all(r[2] == 0 for r in rep2)


def test_skip_needs_all_rows_of_the_group():
    d = 16
    n = 128
    q = _rand((n, 1, d), 17)
    k = _rand((n, 1, d), 18, 0.1)
    v = _rand((n, 1, d), 19)
    k[0] = 40.0 * q[0] / np.linalg.norm(q[0])   # dominates only for row 0's direction
    q[1:32] = -q[0]                              # other rows see key 0 as tiny
    _, rep = fp8_attn_emulated_ref(q, k, v, [0, n], quantize=False, skip=True)
    assert rep[0][2] == 0


def test_groups_restrict_the_work():
    cu = [0, 100]
    q, k, v = _rand((100, 2, 16), 20), _rand((100, 2, 16), 21), _rand((100, 2, 16), 22)
    full, _ = fp8_attn_emulated_ref(q, k, v, cu)
    part, rep = fp8_attn_emulated_ref(q, k, v, cu, groups=[(1, 64)])
    assert np.array_equal(part[64:96, 1], full[64:96, 1])
    assert not part[:, 0].any() and len(rep) == 1


def _bf16_values(shape, seed, std=1.0):
    """float64 values that are exactly bf16 (what the quantiser reads)."""
    a = (std * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)
    bits = a.view(np.uint32)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.view(np.float32).astype(np.float64)


def _exact_e4m3_code(fr):
    """Exact RNE of a Fraction onto the e4m3fn grid (saturating at 448): the
    nearest grid value, ties to the even code (codes of non-negative values
    are their index in the ascending grid)."""
    from fractions import Fraction
    grid = [Fraction(0)] + [Fraction(v) for v in _positive_e4m3_grid()]
    mag = min(abs(fr), Fraction(448))
    best = min(range(len(grid)), key=lambda i: (abs(grid[i] - mag), i % 2))
    return float(grid[best]) * (-1.0 if fr < 0 else 1.0)


def test_codes_are_exact_decisions_for_bf16_inputs():
    """For bf16 x and amax the float64 code RNE(448 x / amax) equals the
    exact rational decision, including exact midpoints (ties to even)."""
    from fractions import Fraction
    x = _bf16_values((64, 1, 128), 21, 1.3)
    x[0, 0, 0] = 4.0                   # a power-of-two amax puts many quotients on midpoints
    codes, scales = quantize_qk_blocks(np.clip(x, -4, 4), [0, 64], 64)
    xs = np.clip(x, -4, 4)
    amax = Fraction(4)
    ties = 0
    for t in range(64):
        for d in range(0, 128, 3):
            q = Fraction(448) * Fraction(float(xs[t, 0, d])) / amax
            want = _exact_e4m3_code(q)
            assert codes[t, 0, d] == want, (t, d, float(q))
            ties += q.denominator <= 2 and abs(q) > 16
    assert ties > 10
    assert scales[0, 0] == 4.0 / 448.0


def test_tie_example_goes_to_even():
    """448 * (-1.4296875) / 3.8125 = -168 exactly, the midpoint of -160 and
    -176: the code is -160 (even mantissa). Dividing by a rounded scale
    amax / 448 instead would land just past the midpoint."""
    x = np.zeros((1, 1, 4))
    x[0, 0, :2] = [-1.4296875, 3.8125]
    codes, scales = quantize_qk_blocks(x, [0, 1], 64)
    assert codes[0, 0, 0] == -160.0 and codes[0, 0, 1] == 448.0
    assert e4m3_round(-1.4296875 / (3.8125 / 448.0)) == -176.0


def test_codes_match_torch_float32_pipeline():
    """The fp32 evaluation (448 x) / amax of bf16 inputs followed by torch's
    float8_e4m3fn cast gives the same codes (448 x is exact in fp32 and one
    correctly rounded division decides)."""
    torch = pytest.importorskip("torch")
    cu = [0, 100, 100, 229]
    x = _bf16_values((229, 3, 128), 22, 1.7)
    codes, scales = quantize_qk_blocks(x, cu, 64)
    for bi, (a, b) in enumerate([(0, 64), (64, 100), (100, 164), (164, 228), (228, 229)]):
        xt = torch.from_numpy(x[a:b].astype(np.float32))
        amax = xt.abs().amax(dim=(0, 2))
        ref = ((xt * 448.0) / amax[None, :, None]).to(torch.float8_e4m3fn).to(torch.float64)
        assert np.array_equal(codes[a:b], ref.numpy())
        assert np.array_equal(scales[bi].astype(np.float32), (amax / 448.0).numpy())
    vc, vs = quantize_v_channels(x, cu)
    for s, (a, b) in enumerate([(0, 100), (100, 100), (100, 229)]):
        if a == b:
            assert (vs[s] == 1.0).all()
            continue
        xt = torch.from_numpy(x[a:b].astype(np.float32))
        amax = xt.abs().amax(dim=0)
        ref = ((xt * 448.0) / amax[None]).to(torch.float8_e4m3fn).to(torch.float64)
        assert np.array_equal(vc[a:b], ref.numpy())


def test_one_tile_matches_direct_formula():
    """A segment of one key tile makes the online softmax a single step:
    written out from the e4m3 definitions (codes from amax, S from the codes
    and scales, P = e4m3(448 p) in the numerator, denominator the sum of the
    unquantised p), the emulation must agree to rounding. The denominator
    summed from the encoded P instead is measurably different, so this pin
    tells the two readings apart."""
    rng = np.random.default_rng(71)
    q, k, v = (np.asarray(rng.standard_normal((60, 1, 128)), dtype=np.float64) for _ in range(3))
    out, _ = fp8_attn_emulated_ref(q, k, v, [0, 60])
    aq, ak = np.abs(q).max(), np.abs(k).max()
    qc, kc = e4m3_round(448 * q[:, 0] / aq), e4m3_round(448 * k[:, 0] / ak)
    s = (qc @ kc.T) * (aq / 448) * (ak / 448) / math.sqrt(128)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    av = np.abs(v[:, 0]).max(axis=0)
    vc = e4m3_round(448 * v[:, 0] / av)
    p8 = e4m3_round(448 * p)
    ref = (p8 @ vc) * (av / 448)[None, :] / (448 * p.sum(axis=1, keepdims=True))
    assert np.max(np.abs(out[:, 0] - ref)) < 1e-12
    other = (p8 @ vc) * (av / 448)[None, :] / p8.sum(axis=1, keepdims=True)
    assert np.max(np.abs(other - ref)) > 1e-6
