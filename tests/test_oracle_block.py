"""Pins of the oracle's DiT block (AdaLN modulation, SwiGLU, gated residuals).

Weights are crafted so that each intermediate has a closed form: one
modulation chunk at a time, identity projections, uniform attention.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import (adaln_modulate_ref, dit_block_ref, dit_block_rows_ref, modulation_ref,
                    rmsnorm, silu, swiglu_ref)

H, D = 2, 8
C = H * D
SPLIT = (2, 2, 4)
EPS = 1e-6


def _rand(shape, seed, std=1.0):
    return std * np.random.default_rng(seed).standard_normal(shape)


def _weights(seed, ffn=C, std=0.3):
    return {
        "w_mod": _rand((6 * C, C), seed + 1, std), "w_qkv": _rand((3 * C, C), seed + 2, std),
        "w_o": _rand((C, C), seed + 3, std), "q_norm": 1 + _rand(D, seed + 4, 0.1),
        "k_norm": 1 + _rand(D, seed + 5, 0.1), "w_gate": _rand((ffn, C), seed + 6, std),
        "w_up": _rand((ffn, C), seed + 7, std), "w_down": _rand((C, ffn), seed + 8, std),
    }


def _case(seed=0, cu=(0, 7, 7, 19)):
    n = cu[-1]
    x = _rand((n, C), seed + 100)
    cond = _rand((len(cu) - 1, C), seed + 101)
    grid = np.random.default_rng(seed + 102).integers(0, 30, size=(n, 3))
    return list(cu), x, cond, grid


def _mod_with_only(chunk, values, b):
    """W_mod, cond giving mod = 0 except chunk `chunk` = values [B, C]."""
    idx = oracle.MOD_CHUNKS.index(chunk)
    w_mod = np.zeros((6 * C, C))
    w_mod[idx * C:(idx + 1) * C, :] = np.eye(C)
    cond = np.asarray(values).reshape(b, C)
    return w_mod, cond


def test_modulation_is_linear_map_of_cond():
    w = _rand((6 * C, C), 1)
    for i in range(C):
        e = np.zeros((1, C))
        e[0, i] = 1.0
        assert np.array_equal(modulation_ref(e, w)[0], w[:, i])


def test_silu_known_values():
    assert silu(0.0) == 0.0
    assert silu(1.0) == pytest.approx(0.7310585786300049, abs=1e-15)
    assert silu(-1.0) == pytest.approx(-0.2689414213699951, abs=1e-15)
    assert silu(40.0) == pytest.approx(40.0, abs=1e-14)
    assert abs(silu(-40.0)) < 1e-15


def test_swiglu_closed_forms():
    h = _rand((9, C), 2)
    assert np.array_equal(swiglu_ref(h, _rand((5, C), 3), np.zeros((5, C))), np.zeros((9, 5)))
    alpha = 1.7
    a = swiglu_ref(h, alpha * np.eye(C), np.eye(C))
    expect = np.vectorize(lambda z: alpha * z * z / (1.0 + math.exp(-alpha * z)))(h)
    assert np.max(np.abs(a - expect)) < 1e-13


def test_adaln_special_cases_and_segment_lookup():
    x = _rand((6, C), 4)
    seg = np.array([0, 0, 1, 1, 1, 2])
    zero = np.zeros((3, C))
    assert np.array_equal(adaln_modulate_ref(x, zero, zero, seg, EPS), rmsnorm(x, EPS))
    shift = np.arange(3)[:, None] * np.ones((3, C))
    out = adaln_modulate_ref(x, shift, -np.ones((3, C)), seg, EPS)
    assert np.array_equal(out, shift[seg])            # scale = -1 removes the norm term
    out = adaln_modulate_ref(x, zero, np.ones((3, C)), seg, EPS)
    assert np.allclose(out, 2 * rmsnorm(x, EPS), atol=1e-15)


def test_zero_gates_give_identity_bitwise():
    cu, x, cond, grid = _case(1)
    w = _weights(1)
    w_mod = w["w_mod"].copy()
    w_mod[2 * C:3 * C] = 0.0       # gate1
    w_mod[5 * C:6 * C] = 0.0       # gate2
    w["w_mod"] = w_mod
    r = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    assert np.array_equal(r["x1"], x)
    assert np.array_equal(r["x2"], x)


@pytest.mark.parametrize("chunk", ["shift1", "scale1", "shift2", "scale2"])
def test_modulation_chunk_order(chunk):
    cu, x, _, grid = _case(2)
    b = len(cu) - 1
    vals = _rand((b, C), 3)
    w = _weights(2)
    w["w_mod"], cond = _mod_with_only(chunk, vals, b)
    r = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    seg = oracle.segment_ids(cu)
    # all gates are zero in this construction, so x1 == x2 == x
    assert np.array_equal(r["x2"], x)
    if chunk == "shift1":
        assert np.allclose(r["h"], rmsnorm(x, EPS) + vals[seg], atol=1e-14)
    elif chunk == "scale1":
        assert np.allclose(r["h"], rmsnorm(x, EPS) * (1 + vals[seg]), atol=1e-14)
    elif chunk == "shift2":
        assert np.allclose(r["h2"], rmsnorm(x, EPS) + vals[seg], atol=1e-14)
    else:
        assert np.allclose(r["h2"], rmsnorm(x, EPS) * (1 + vals[seg]), atol=1e-14)


def test_gate_chunks_and_uniform_attention_closed_form():
    # q = k = 0 -> uniform attention; v = h; W_o = I; gate1 = g1; gate2 = 0:
    # x1 = x + g1 * (segment mean of h), h = RMSNorm(x) (no shift/scale).
    cu, x, _, grid = _case(3, cu=(0, 5, 12, 12, 20))
    b = len(cu) - 1
    g1 = _rand((b, C), 4)
    w = _weights(3)
    w["w_mod"], cond = _mod_with_only("gate1", g1, b)
    w_qkv = np.zeros((3 * C, C))
    w_qkv[2 * C:] = np.eye(C)
    w["w_qkv"] = w_qkv
    w["w_o"] = np.eye(C)
    r = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    hn = rmsnorm(x, EPS)
    expect = x.copy()
    for s in range(b):
        a, e = cu[s], cu[s + 1]
        if e > a:
            expect[a:e] += g1[s] * hn[a:e].mean(axis=0)
    assert np.max(np.abs(r["x1"] - expect)) < 1e-13
    assert np.array_equal(r["x2"], r["x1"])


def test_mlp_branch_closed_form():
    # gate2 = 1 only; W_gate = alpha I, W_up = I, W_down = I: x2 = x1 + silu(alpha h2) h2
    cu, x, _, grid = _case(4)
    b = len(cu) - 1
    w = _weights(4)
    w["w_mod"], cond = _mod_with_only("gate2", np.ones((b, C)), b)
    alpha = 0.8
    w["w_gate"], w["w_up"], w["w_down"] = alpha * np.eye(C), np.eye(C), np.eye(C)
    r = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    h2 = rmsnorm(x, EPS)
    expect = x + np.vectorize(lambda z: alpha * z * z / (1.0 + math.exp(-alpha * z)))(h2)
    assert np.max(np.abs(r["x2"] - expect)) < 1e-13


def test_segment_swap_permutes_outputs():
    cu = [0, 6, 17]
    _, x, cond, grid = _case(5, cu=tuple(cu))
    w = _weights(5)
    r = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    perm = np.r_[6:17, 0:6]
    r2 = dit_block_ref(x[perm], cond[::-1], w, [0, 11, 17], grid[perm], H, D, SPLIT, eps=EPS)
    assert np.max(np.abs(r2["x2"] - r["x2"][perm])) < 1e-13


def test_token_permutation_inside_segment_with_positions():
    cu = [0, 13]
    _, x, cond, grid = _case(6, cu=tuple(cu))
    w = _weights(6)
    r = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    perm = np.random.default_rng(7).permutation(13)
    r2 = dit_block_ref(x[perm], cond, w, cu, grid[perm], H, D, SPLIT, eps=EPS)
    assert np.max(np.abs(r2["x2"] - r["x2"][perm])) < 1e-13


def test_sampled_rows_path_equals_full_path():
    cu, x, cond, grid = _case(7, cu=(0, 9, 9, 31))
    w = _weights(7, ffn=24)
    full = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    rows = np.array([0, 8, 9, 20, 30])
    part = dit_block_rows_ref(x, cond, w, cu, grid, H, D, SPLIT, rows, eps=EPS, token_chunk=4)
    for key in ("h", "o", "x1", "h2", "a", "x2"):
        assert np.max(np.abs(part[key] - full[key][rows])) < 1e-12, key


def test_bf16_round_ties_and_torch_cast():
    from oracle import bf16_round
    assert bf16_round(1.0 + 2.0 ** -8) == 1.0                    # tie -> even
    assert bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie -> even
    assert bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert bf16_round(-3.0) == -3.0 and bf16_round(0.0) == 0.0
    torch = pytest.importorskip("torch")
    a = np.random.default_rng(9).standard_normal(50000).astype(np.float32)
    a[:100] *= 1e-30
    a[100:200] *= 1e30
    t = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(a.astype(np.float64)), t)


def test_storage_emulation_rounds_every_boundary_and_stays_close():
    from oracle import bf16_round
    cu, x, cond, grid = _case(8, cu=(0, 9, 20))
    x = bf16_round(x)
    w = _weights(8, ffn=24)
    ex = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS)
    em = dit_block_ref(x, cond, w, cu, grid, H, D, SPLIT, eps=EPS, emulate_bf16_storage=True)
    for key in ("h", "qkv", "q", "k", "o", "x1", "h2", "a", "x2"):
        assert np.array_equal(bf16_round(em[key]), em[key]), key
        assert oracle.rel_frobenius(em[key], ex[key]) < 1e-2, key
    assert np.array_equal(em["mod"].astype(np.float32).astype(np.float64), em["mod"])
    rows = np.array([0, 5, 19])
    part = dit_block_rows_ref(x, cond, w, cu, grid, H, D, SPLIT, rows, eps=EPS,
                              emulate_bf16_storage=True, token_chunk=4)
    for key in ("h", "o", "x1", "h2", "a", "x2"):
        assert np.max(np.abs(part[key] - em[key][rows])) < 1e-12, key
