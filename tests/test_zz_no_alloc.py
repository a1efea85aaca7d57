"""h3_attn_varlen_noalloc (no workspace argument; the library's fixed
per-GPU scratch array) against h3_attn_varlen on the same inputs, called
through the C ABI: the outputs must be bit-identical (both run the same
kernels) and within the bf16 bar of the float64 oracle, on two calls in a
row with the second input smaller, for the bf16 and the fp8 path; sizes
beyond the fixed scratch are rejected before any launch."""
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


def _inputs(lens, heads, d, seed):
    cu = h3synth.cu_from_lengths(lens)
    n = int(cu[-1])
    return cu, h3synth.attention_inputs(cu, np.zeros((n, 3), np.int32), heads, d, seed=seed)


@pytest.mark.parametrize("precision,cases", [
    # 8 heads: work items dealt to the XCDs by head, located through the
    # schedule's tile prefix, which lives in the scratch / workspace
    ("bf16", [([900, 0, 517], 8, 128), ([300, 65], 2, 64)]),
    ("fp8", [([700, 129, 1], 3, 128), ([200], 2, 128)]),
])
def test_noalloc_equals_workspace_entry_point(dev, ops, precision, cases):
    import torch
    for i, (lens, heads, d) in enumerate(cases):
        announce(f"noalloc {precision} call {i + 1} lens={lens} H={heads} D={d}")
        cu, inp = _inputs(lens, heads, d, seed=600 + i)
        q, k, v = (to_dev_bf16(a, dev) for a in (inp.q, inp.k, inp.v))
        cu_d = to_dev_i32(cu, dev)
        n_items = ops.attn_num_items(cu, heads)
        skip = precision == "fp8"
        c_ws = torch.full((n_items,), -1, dtype=torch.int32, device=dev) if skip else None
        c_na = torch.full((n_items,), -1, dtype=torch.int32, device=dev) if skip else None
        ref_out = ops.attn_varlen(q, k, v, cu_d, cu, precision=precision, skip_softmax=skip,
                                  skip_counts=c_ws)
        out = torch.full_like(ref_out, float("nan"))
        ops.attn_varlen_noalloc(q, k, v, cu_d, cu, out, precision=precision, skip_softmax=skip,
                                skip_counts=c_na)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_of(out), bf16_bits_of(ref_out))
        if skip:
            assert torch.equal(c_na, c_ws)
        if precision == "bf16":
            ref = oracle.attn_varlen_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu)
        else:
            ref, _ = oracle.fp8_attn_emulated_ref(inp.q.f32, inp.k.f32, inp.v.f32, cu, skip=True)
        compare(to_np(out), ref, f"noalloc {precision} call {i + 1}",
                scaled_abs=2e-2 if precision == "bf16" else 5e-2)


def test_noalloc_rejects_sizes_beyond_its_scratch(dev, ops):
    """fp8 at 8,000 tokens x 24 heads needs about 72 MiB of scratch, more
    than the fixed 64 MiB: H3_ERR_WORKSPACE_TOO_SMALL, nothing written."""
    import torch
    announce("noalloc fp8 beyond the fixed scratch")
    n, heads = 8000, 24
    cu = np.array([0, n], np.int32)
    assert ops.attn_workspace_bytes(cu, n, heads, 128, "fp8") > (64 << 20)
    q = torch.zeros((n, heads, 128), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 3.0)
    with pytest.raises(Exception) as e:
        ops.attn_varlen_noalloc(q, q, q, to_dev_i32(cu, dev), cu, out, precision="fp8")
    assert "WORKSPACE_TOO_SMALL" in str(e.value) or "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
