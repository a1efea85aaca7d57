"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every entry point that include/h3dit.h
declares, reject malformed arguments before enqueuing anything, and build
the attention work list exactly as the oracle's schedule specification.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_packed_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3dit.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libh3dit.so is not built (run __graft_entry__.build())")
    return L.lib()


def _header_symbols():
    text = open(HEADER).read()
    return re.findall(r"H3_API\s+[\w\s\*]+?\b(h3_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported(lib):
    names = _header_symbols()
    assert len(names) >= 15
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_only_the_c_abi_is_exported(lib):
    out = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read().split("\n")
    exported = {ln.split()[-1] for ln in out if " T " in ln}
    assert {n for n in exported if n.startswith("h3_")} == set(L.EXPORTS)
    assert not any(n.startswith("_ZN2h3") for n in exported)


def test_status_strings_and_version(lib):
    assert lib.h3_abi_version() == 1
    assert lib.h3_status_string(0) == b"H3_OK"
    assert lib.h3_status_string(3) == b"H3_ERR_WORKSPACE_TOO_SMALL"
    assert lib.h3_status_string(99) == b"H3_ERR_UNKNOWN"


def _cu(arr):
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
    return a, a.ctypes.data_as(C.c_void_p)


def _attn(lib, cu_list, n, heads=2, d=128, ws_bytes=1 << 20, opts=None, strides=None,
          q=0x1000, null_cu_dev=False):
    a, p = _cu(cu_list)
    st = strides or (heads * d,) * 4
    return lib.h3_attn_varlen(C.c_void_p(q), C.c_void_p(0x2000), C.c_void_p(0x3000),
                              C.c_void_p(0x4000), *st, None if null_cu_dev else C.c_void_p(0x5000),
                              p, a.size - 1, n, heads, d, None if opts is None else C.byref(opts),
                              C.c_void_p(0x10000), ws_bytes, None)


@pytest.mark.parametrize("cu,n", [([1, 5], 5), ([0, 5, 3], 3), ([0, 4], 5), ([0, -1, 0], 0)])
def test_attention_rejects_malformed_cu_seqlens(lib, cu, n):
    assert _attn(lib, cu, n) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_last_error_message()


def test_attention_argument_errors(lib):
    assert _attn(lib, [0, 10], 10, d=96) == L.H3_ERR_UNSUPPORTED
    assert _attn(lib, [0, 10], 10, heads=0) == L.H3_ERR_INVALID_ARGUMENT
    assert _attn(lib, [0, 10], 10, ws_bytes=0) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert _attn(lib, [0, 10], 10, strides=(100, 256, 256, 256)) == L.H3_ERR_INVALID_ARGUMENT
    assert _attn(lib, [0, 10], 10, strides=(260, 256, 256, 256)) == L.H3_ERR_UNSUPPORTED
    assert _attn(lib, [0, 10], 10, q=0x1001) == L.H3_ERR_UNSUPPORTED
    assert _attn(lib, [0, 10], 10, q=0) == L.H3_ERR_INVALID_ARGUMENT
    assert _attn(lib, [0, 10], 10, null_cu_dev=True) == L.H3_ERR_INVALID_ARGUMENT
    bad = L.AttnOpts(7, 0, 8.0, 0.0, None)
    assert _attn(lib, [0, 10], 10, opts=bad) == L.H3_ERR_INVALID_ARGUMENT
    skip_bf16 = L.AttnOpts(L.H3_ATTN_BF16, 1, 8.0, 0.0, None)
    assert _attn(lib, [0, 10], 10, opts=skip_bf16) == L.H3_ERR_UNSUPPORTED
    neg = L.AttnOpts(L.H3_ATTN_BF16, 0, 8.0, -1.0, None)
    assert _attn(lib, [0, 10], 10, opts=neg) == L.H3_ERR_INVALID_ARGUMENT
    fp8_64 = L.AttnOpts(L.H3_ATTN_FP8_E4M3, 0, 8.0, 0.0, None)
    assert _attn(lib, [0, 10], 10, d=64, opts=fp8_64) == L.H3_ERR_UNSUPPORTED
    # empty input is a no-op and needs nothing
    assert _attn(lib, [0, 0, 0], 0, ws_bytes=0) == L.H3_OK
    assert _attn(lib, [0], 0, ws_bytes=0) == L.H3_OK


def _attn_noalloc(lib, cu_list, n, heads=2, d=128, opts=None, q=0x1000):
    a, p = _cu(cu_list)
    st = (heads * d,) * 4
    return lib.h3_attn_varlen_noalloc(C.c_void_p(q), C.c_void_p(0x2000), C.c_void_p(0x3000),
                                      C.c_void_p(0x4000), *st, C.c_void_p(0x5000), p, a.size - 1, n,
                                      heads, d, None if opts is None else C.byref(opts), None)


def test_attention_noalloc_argument_errors(lib):
    """The no-workspace variant applies the same checks before anything
    else, and rejects sizes beyond its fixed 64 MiB scratch before touching
    the device."""
    assert _attn_noalloc(lib, [1, 5], 5) == L.H3_ERR_INVALID_ARGUMENT
    assert _attn_noalloc(lib, [0, 10], 10, d=96) == L.H3_ERR_UNSUPPORTED
    assert _attn_noalloc(lib, [0, 10], 10, q=0) == L.H3_ERR_INVALID_ARGUMENT
    fp8 = L.AttnOpts(L.H3_ATTN_FP8_E4M3, 0, 8.0, 0.0, None)
    assert lib.h3_attn_varlen_workspace_size(1, 8000, 24, 128, C.byref(fp8)) > (64 << 20)
    assert _attn_noalloc(lib, [0, 8000], 8000, heads=24, opts=fp8) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert b"64" in lib.h3_last_error_message() or b"scratch" in lib.h3_last_error_message()
    assert _attn_noalloc(lib, [0, 0], 0) == L.H3_OK


def test_workspace_sizes(lib):
    small = lib.h3_attn_varlen_workspace_size(1, 100, 2, 128, None)
    big = lib.h3_attn_varlen_workspace_size(1, 100000, 24, 128, None)
    assert 0 < small < big and small % 256 == 0
    assert lib.h3_attn_varlen_workspace_size(1, 100, 2, 96, None) == 0
    # capacity covers the worst case over all cu_seqlens with these sizes
    for b, n in [(1, 1), (3, 3), (5, 700), (64, 64 * 129)]:
        need = lib.h3_attn_varlen_workspace_size(b, n, 4, 64, None)
        bm = L.H3_ATTN_BLOCK_M
        assert need >= 16 * 4 * ((n + b * (bm - 1)) // bm)
    dims = L.DitDims(3072, 24, 128, 8192, (C.c_int32 * 3)(32, 48, 48), 1e4, 1e-6)
    ws = lib.h3_dit_block_workspace_size(C.byref(dims), 1, 57960)
    n, c = 57960, 3072
    assert ws >= 2 * n * (c * 7 + 8192)  # h, qkv, o, x1, h2 and a
    bad = L.DitDims(3072, 24, 128, 8192, (C.c_int32 * 3)(32, 48, 46), 1e4, 1e-6)
    assert lib.h3_dit_block_workspace_size(C.byref(bad), 1, 100) == 0


def test_block_argument_errors(lib):
    a, p = _cu([0, 10])
    w = L.DitWeights(*([0x1000] * 8))

    def call(dims, ws=1 << 40, x=0x1000, out=0x2000):
        return lib.h3_dit_block_forward(C.c_void_p(x), C.c_void_p(out), C.c_void_p(0x3000),
                                        C.byref(w), C.byref(dims), C.c_void_p(0x4000), p, 1, 10,
                                        C.c_void_p(0x5000), None, C.c_void_p(0x100000), ws, None)

    split = (C.c_int32 * 3)(32, 48, 48)
    assert call(L.DitDims(3072, 24, 128, 8192, split, 1e4, 1e-6), ws=0) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert call(L.DitDims(3072, 24, 64, 8192, (C.c_int32 * 3)(16, 24, 24), 1e4, 1e-6)) == L.H3_ERR_INVALID_ARGUMENT
    assert call(L.DitDims(3072, 24, 128, 8100, split, 1e4, 1e-6)) == L.H3_ERR_UNSUPPORTED
    assert call(L.DitDims(3072, 24, 128, 8192, (C.c_int32 * 3)(31, 49, 48), 1e4, 1e-6)) == L.H3_ERR_INVALID_ARGUMENT
    assert call(L.DitDims(3072, 24, 128, 8192, split, -1.0, 1e-6)) == L.H3_ERR_INVALID_ARGUMENT
    assert call(L.DitDims(3072, 24, 128, 8192, split, 1e4, 1e-6), x=0x2000) == L.H3_ERR_INVALID_ARGUMENT
    assert call(L.DitDims(2880, 24, 120, 8192, split, 1e4, 1e-6)) == L.H3_ERR_UNSUPPORTED


def test_op_argument_errors(lib):
    a, p = _cu([0, 10])
    split = (C.c_int32 * 3)(16, 24, 24)
    bad_split = (C.c_int32 * 3)(16, 24, 26)
    X = C.c_void_p(0x1000)
    assert lib.h3_qk_rmsnorm_rope(X, X, 256, 256, X, X, X, 10, 4, 64, bad_split, 1e4, 1e-6, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_qk_rmsnorm_rope(X, X, 256, 256, X, X, X, 10, 4, 80, split, 1e4, 1e-6, None) == L.H3_ERR_UNSUPPORTED
    assert lib.h3_qk_rmsnorm_rope(X, X, 100, 256, X, X, X, 10, 4, 64, split, 1e4, 1e-6, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_qk_rmsnorm_rope(None, X, 256, 256, X, X, X, 10, 4, 64, split, 1e4, 1e-6, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_qk_rmsnorm_rope(X, X, 256, 256, X, X, X, 10, 4, 64, split, 1e4, -1.0, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_modulation(X, X, X, 1, 3000, None) == L.H3_ERR_UNSUPPORTED
    assert lib.h3_modulation(X, None, X, 1, 3072, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_adaln_rmsnorm_modulate(X, X, X, X, 6 * 3072, X, p, 1, 11, 3072, 1e-6, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_adaln_rmsnorm_modulate(X, X, X, X, 100, X, p, 1, 10, 3072, 1e-6, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_linear_bf16(X, X, X, 10, 100, 64, None) == L.H3_ERR_UNSUPPORTED
    assert lib.h3_linear_bf16(X, X, X, 10, 128, 60, None) == L.H3_ERR_UNSUPPORTED
    assert lib.h3_linear_bf16(X, X, X, -1, 128, 64, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_linear_bf16(X, X, X, 0, 128, 64, None) == L.H3_OK
    assert lib.h3_linear_swiglu_bf16(X, X, X, X, 10, 90, 64, None) == L.H3_ERR_UNSUPPORTED
    assert lib.h3_linear_gated_residual_bf16(X, X, X, X, 128, X, 11, 128, 64, X, p, 1, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_linear_gated_residual_bf16(X, X, X, X, 64, X, 10, 128, 64, X, p, 1, None) == L.H3_ERR_INVALID_ARGUMENT


ADVERSARIAL = [0, 1, 2, 63, 64, 65, 127, 128, 129]


@pytest.mark.parametrize("lens,heads,block_m", [
    ([704, 512], 4, 128),
    ([32260], 24, 128),
    ([57960], 24, 128),
    ([93740], 24, 128),
    (ADVERSARIAL, 3, 128),
    (ADVERSARIAL[::-1] + [65, 64], 2, 64),
    ([5, 5, 5, 0, 5], 1, 2),
    ([], 4, 128),
    ([32260], 24, 256),
    ([57960], 24, 256),
    ([93740], 24, 256),
    ([0, 1, 255, 256, 257, 511, 512, 513, 128, 129, 0], 3, 256),
])
def test_host_schedule_matches_spec(lib, lens, heads, block_m):
    from audio_diffusion_transformer_packed_amd.ops import build_schedule_host
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    got = build_schedule_host(cu, heads, block_m)
    ref = oracle.schedule_ref(cu, heads, block_m)
    assert got.dtype == np.int32 and np.array_equal(got, ref)


def test_host_schedule_errors(lib):
    a, p = _cu([0, 3, 2])
    cnt = C.c_int64(0)
    assert lib.h3_build_schedule_host(p, 2, 1, 128, None, 0, C.byref(cnt)) == L.H3_ERR_INVALID_ARGUMENT
    a, p = _cu([0, 300])
    assert lib.h3_build_schedule_host(p, 1, 2, 128, None, 0, C.byref(cnt)) == L.H3_OK
    assert cnt.value == 6
    buf = np.zeros((5, 4), np.int32)
    assert lib.h3_build_schedule_host(p, 1, 2, 128, buf.ctypes.data_as(C.c_void_p), 5,
                                      C.byref(cnt)) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert lib.h3_build_schedule_host(p, 1, 2, 0, None, 0, C.byref(cnt)) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_build_schedule_host(p, 1, 2, 128, None, 0, None) == L.H3_ERR_INVALID_ARGUMENT


def test_bookkeeping_argument_errors(lib):
    a, p = _cu([0, 300])
    X = C.c_void_p(0x1000)
    assert lib.h3_varlen_bookkeeping(X, p, 1, 300, 2, 128, X, X, X, 5, X, 1024, None) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert lib.h3_varlen_bookkeeping(X, p, 1, 300, 2, 128, X, X, X, 6, X, 0, None) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert lib.h3_varlen_bookkeeping(None, p, 1, 300, 2, 128, X, X, X, 6, X, 1024, None) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_varlen_bookkeeping(X, p, 1, 301, 2, 128, X, X, X, 6, X, 1024, None) == L.H3_ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="build the HIP library"):
        L.lib()


def test_fp8_num_tiles_and_workspace(lib):
    cu, cup = _cu([0, 1, 65, 65, 193])
    t = C.c_int64(-1)
    assert lib.h3_fp8_num_tiles(cup, 4, C.byref(t)) == L.H3_OK and t.value == 4
    bad, badp = _cu([0, 5, 3])
    assert lib.h3_fp8_num_tiles(badp, 2, C.byref(t)) == L.H3_ERR_INVALID_ARGUMENT
    assert lib.h3_fp8_num_tiles(cup, 4, None) == L.H3_ERR_INVALID_ARGUMENT
    small = lib.h3_fp8_quantize_workspace_size(1, 100, 2)
    big = lib.h3_fp8_quantize_workspace_size(1, 100000, 24)
    assert 0 < small < big and small % 256 == 0
    assert lib.h3_fp8_quantize_workspace_size(1, 100, 0) == 0


def test_fp8_quantize_argument_errors(lib):
    """Every case is rejected on the host before any launch (fake aligned
    device addresses are never dereferenced)."""
    cu, cup = _cu([0, 10])
    fake = C.c_void_p(1 << 20)
    ws_ok = lib.h3_fp8_quantize_workspace_size(1, 10, 2)

    def call(d=128, q=fake, stride=256, ws=ws_ok, k8=fake, n=10, cu_p=cup, align=0):
        qq = C.c_void_p(q.value + align) if q is not None and q.value else q
        return lib.h3_fp8_quantize(qq, fake, fake, stride, stride, stride, fake, cu_p, 1, n, 2, d,
                                   fake, k8, fake, fake, fake, fake, fake, ws, None)
    assert call(d=64) == L.H3_ERR_UNSUPPORTED
    assert call(q=C.c_void_p(0)) == L.H3_ERR_INVALID_ARGUMENT
    assert call(k8=C.c_void_p(0)) == L.H3_ERR_INVALID_ARGUMENT
    assert call(stride=200) == L.H3_ERR_INVALID_ARGUMENT
    assert call(stride=260) == L.H3_ERR_UNSUPPORTED
    assert call(align=8) == L.H3_ERR_UNSUPPORTED
    assert call(ws=ws_ok - 1) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert call(n=11) == L.H3_ERR_INVALID_ARGUMENT            # cu[B] != total_tokens
    zcu, zcup = _cu([0, 0])
    assert call(n=0, cu_p=zcup) == L.H3_OK                    # nothing to do, nothing launched


def _bsa(lib, cu, n, d=128, heads=2, sparsity=0.8, ws_bytes=1 << 30, lists=0):
    cu_arr = (C.c_int32 * len(cu))(*cu)
    return lib.h3_attn_block_sparse(C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x3000),
                                    C.c_void_p(0x4000), heads * d, heads * d, heads * d, heads * d,
                                    C.c_void_p(0x5000), cu_arr, len(cu) - 1, n, heads, d,
                                    C.c_float(0.0), C.c_float(sparsity), C.c_void_p(lists),
                                    C.c_void_p(0x10000), ws_bytes, None)


def test_block_sparse_argument_errors_and_sizes(lib):
    """Host-side checks of the block-sparse entry points (no GPU call is
    reached: every case fails validation first)."""
    assert _bsa(lib, [0, 10], 10, d=64) == L.H3_ERR_UNSUPPORTED
    assert _bsa(lib, [0, 10], 10, sparsity=1.0) == L.H3_ERR_INVALID_ARGUMENT
    assert _bsa(lib, [0, 10], 10, sparsity=-0.1) == L.H3_ERR_INVALID_ARGUMENT
    assert _bsa(lib, [0, 10], 10, ws_bytes=0) == L.H3_ERR_WORKSPACE_TOO_SMALL
    assert _bsa(lib, [0, 10], 10, lists=0x1002) == L.H3_ERR_INVALID_ARGUMENT
    big = 4096 * 64 + 1
    assert _bsa(lib, [0, big], big, ws_bytes=1 << 40) == L.H3_ERR_UNSUPPORTED
    assert _bsa(lib, [0, 5, 3], 3) == L.H3_ERR_INVALID_ARGUMENT
    ws = lib.h3_attn_block_sparse_workspace_size
    assert ws(1, 1000, 2, 64, C.c_float(0.8)) == 0 and ws(1, 1000, 2, 128, C.c_float(1.0)) == 0
    assert ws(1, 57960, 24, 128, C.c_float(0.8)) > ws(1, 57960, 24, 128, C.c_float(0.9)) > 0
    stride = C.c_int64(0)
    cu = (C.c_int32 * 4)(0, 640, 640, 6400)                    # 10 and 90 key blocks
    assert lib.h3_attn_block_sparse_list_stride(cu, 3, C.c_float(0.8), C.byref(stride)) == L.H3_OK
    assert stride.value == 18                                  # 90 - floor(72.0)
    assert lib.h3_attn_block_sparse_list_stride(cu, 3, C.c_float(0.0), C.byref(stride)) == L.H3_OK
    assert stride.value == 90


def test_dense_fallback_helper_matches_oracle():
    from audio_diffusion_transformer_packed_amd import ops
    import oracle
    for start, end in [(8, 13), (8, 12), (0, 13), (0, 0), (50, 0)]:
        for s in range(50):
            assert ops.dense_attention_step(s, 50, start, end) == oracle.dense_fallback(s, 50, start, end)


def test_block_mx_bsa_sizes(lib):
    split = (C.c_int32 * 3)(32, 48, 48)
    dims = L.DitDims(3072, 24, 128, 8192, split, 1e4, 1e-6)
    ws = lib.h3_dit_block_mx_bsa_workspace_size
    dense = lib.h3_dit_block_mx_workspace_size(C.byref(dims), 1, 57960)
    sparse = ws(C.byref(dims), 1, 57960, C.c_float(0.8))
    assert dense > 0 and sparse > 0 and sparse != dense
    assert ws(C.byref(dims), 1, 57960, C.c_float(1.0)) == 0
    dims64 = L.DitDims(3072, 48, 64, 8192, (C.c_int32 * 3)(16, 24, 24), 1e4, 1e-6)
    assert ws(C.byref(dims64), 1, 57960, C.c_float(0.8)) == 0
