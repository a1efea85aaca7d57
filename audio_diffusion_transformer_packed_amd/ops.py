"""Python binding of the HIP library: argument marshalling only.

Each function takes torch tensors (device memory owned by PyTorch), checks
dtypes and layouts, and calls the C ABI entry point of the same name on the
current torch stream. Every step of the computation runs in the library's
HIP kernels; this module computes nothing itself. Workspaces are allocated
from torch's caching allocator when the caller does not pass one.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib as L
from ._lib import AttnOpts, DitDims, DitMxWeights, DitTaps, DitWeights, MxMatrix, check, lib

BF16 = torch.bfloat16


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _host_cu(cu_host) -> np.ndarray:
    if isinstance(cu_host, torch.Tensor):
        cu_host = cu_host.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu_host, dtype=np.int32))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _token_view(t: torch.Tensor, name: str, heads: int, head_dim: int) -> int:
    """Token stride (elements) of a [N, H, D] view with contiguous heads."""
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != head_dim:
        raise ValueError(f"{name} must be [N, {heads}, {head_dim}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != head_dim:
        raise ValueError(f"{name} must have contiguous heads (strides (*, {head_dim}, 1))")
    return t.stride(0)


# --------------------------------------------------------------------------
# Schedule
# --------------------------------------------------------------------------

def build_schedule_host(cu_host, num_heads: int, block_m: int = L.H3_ATTN_BLOCK_M) -> np.ndarray:
    cu = _host_cu(cu_host)
    count = C.c_int64(0)
    check(lib().h3_build_schedule_host(cu.ctypes.data_as(C.c_void_p), cu.size - 1, num_heads,
                                       block_m, None, 0, C.byref(count)))
    items = np.zeros((count.value, 4), dtype=np.int32)
    check(lib().h3_build_schedule_host(cu.ctypes.data_as(C.c_void_p), cu.size - 1, num_heads,
                                       block_m, items.ctypes.data_as(C.c_void_p), count.value,
                                       C.byref(count)))
    return items


def varlen_bookkeeping(cu_seqlens: torch.Tensor, cu_host, num_heads: int,
                       block_m: int = L.H3_ATTN_BLOCK_M) -> Tuple[torch.Tensor, ...]:
    """Device seg_id [N], tile_cu [B+1] and work list [items, 4]."""
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    cu = _host_cu(cu_host)
    b, n = cu.size - 1, int(cu[-1])
    dev = cu_seqlens.device
    count = C.c_int64(0)
    check(lib().h3_build_schedule_host(cu.ctypes.data_as(C.c_void_p), b, num_heads, block_m,
                                       None, 0, C.byref(count)))
    seg_id = torch.empty(n, dtype=torch.int32, device=dev)
    tile_cu = torch.empty(b + 1, dtype=torch.int32, device=dev)
    items = torch.empty((max(count.value, 1), 4), dtype=torch.int32, device=dev)
    ws = _workspace(lib().h3_varlen_bookkeeping_workspace_size(b), dev, None)
    check(lib().h3_varlen_bookkeeping(_ptr(cu_seqlens), cu.ctypes.data_as(C.c_void_p), b, n,
                                      num_heads, block_m, _ptr(seg_id), _ptr(tile_cu),
                                      _ptr(items), count.value, _ptr(ws), ws.numel(),
                                      _stream(dev)))
    return seg_id, tile_cu, items[:count.value]


def attn_num_items(cu_host, num_heads: int) -> int:
    cu = _host_cu(cu_host)
    count = C.c_int64(0)
    check(lib().h3_attn_varlen_num_items(cu.ctypes.data_as(C.c_void_p), cu.size - 1, num_heads,
                                         C.byref(count)))
    return count.value


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                cu_host, out: Optional[torch.Tensor] = None, precision: str = "bf16",
                skip_softmax: bool = False, skip_threshold: float = 8.0,
                softmax_scale: float = 0.0, skip_counts: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Varlen attention over packed segments; q, k, v, out are [N, H, D] bf16."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, BF16, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n, heads, d = q.shape
    if out is None:
        out = torch.empty((n, heads, d), dtype=BF16, device=dev)
    _need(out, "out", BF16, dev)
    strides = [_token_view(t, nm, heads, d) for nm, t in (("q", q), ("k", k), ("v", v), ("out", out))]
    cu = _host_cu(cu_host)
    prec = {"bf16": L.H3_ATTN_BF16, "fp8": L.H3_ATTN_FP8_E4M3}[precision]
    if skip_counts is not None:
        _need(skip_counts, "skip_counts", torch.int32, dev)
    opts = AttnOpts(prec, int(skip_softmax), float(skip_threshold), float(softmax_scale),
                    None if skip_counts is None else skip_counts.data_ptr())
    nbytes = lib().h3_attn_varlen_workspace_size(cu.size - 1, n, heads, d, C.byref(opts))
    ws = _workspace(nbytes, dev, workspace)
    check(lib().h3_attn_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), *strides, _ptr(cu_seqlens),
                               cu.ctypes.data_as(C.c_void_p), cu.size - 1, n, heads, d,
                               C.byref(opts), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def attn_varlen_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                        cu_host, out: torch.Tensor, precision: str = "bf16",
                        skip_softmax: bool = False, skip_threshold: float = 8.0,
                        softmax_scale: float = 0.0,
                        skip_counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """attn_varlen through h3_attn_varlen_noalloc: no workspace, the
    library's fixed per-GPU scratch instead; `out` must be given, so the
    call allocates nothing."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _need(t, name, BF16, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n, heads, d = q.shape
    strides = [_token_view(t, nm, heads, d) for nm, t in (("q", q), ("k", k), ("v", v), ("out", out))]
    cu = _host_cu(cu_host)
    prec = {"bf16": L.H3_ATTN_BF16, "fp8": L.H3_ATTN_FP8_E4M3}[precision]
    if skip_counts is not None:
        _need(skip_counts, "skip_counts", torch.int32, dev)
    opts = AttnOpts(prec, int(skip_softmax), float(skip_threshold), float(softmax_scale),
                    None if skip_counts is None else skip_counts.data_ptr())
    with torch.cuda.device(dev):       # the library looks up the scratch of the current device
        check(lib().h3_attn_varlen_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), *strides,
                                           _ptr(cu_seqlens), cu.ctypes.data_as(C.c_void_p),
                                           cu.size - 1, n, heads, d, C.byref(opts), _stream(dev)))
    return out


def fp8_num_tiles(cu_host) -> int:
    """T = sum over segments of ceil(L_s / 64): the key tiles of the fp8 layouts."""
    cu = _host_cu(cu_host)
    count = C.c_int64(0)
    check(lib().h3_fp8_num_tiles(cu.ctypes.data_as(C.c_void_p), cu.size - 1, C.byref(count)))
    return count.value


def attn_workspace_bytes(cu_host, total_tokens: int, num_heads: int, head_dim: int,
                         precision: str = "bf16") -> int:
    """Workspace bytes h3_attn_varlen needs for these sizes and precision."""
    cu = _host_cu(cu_host)
    prec = {"bf16": L.H3_ATTN_BF16, "fp8": L.H3_ATTN_FP8_E4M3}[precision]
    opts = AttnOpts(prec, 0, 0.0, 0.0, None)
    return lib().h3_attn_varlen_workspace_size(cu.size - 1, total_tokens, num_heads, head_dim,
                                               C.byref(opts))


def fp8_quantize(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                 cu_host, out: Optional[Dict[str, torch.Tensor]] = None,
                 workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """e4m3 codes and scales of q, k, v [N, H, 128] bf16 (layouts in h3dit.h):
    q8 [N, H, 128], k8 [H, T, 64, 128], v8t [H, T, 128, 64] (uint8),
    q_scale / k_scale [T, H], v_scale [B, H, 128] (float32). `out` may hold
    buffers of those shapes from an earlier call."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, BF16, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n, heads, d = q.shape
    strides = [_token_view(t, nm, heads, d) for nm, t in (("q", q), ("k", k), ("v", v))]
    cu = _host_cu(cu_host)
    b = cu.size - 1
    t = fp8_num_tiles(cu)
    u8 = torch.uint8
    if out is not None:
        _need(out["q8"], "q8", u8, dev)
        if tuple(out["k8"].shape) != (heads, t, L.H3_FP8_QK_BLOCK, d):
            raise ValueError("out buffers do not match these sizes")
    out = out if out is not None else {
        "q8": torch.empty((n, heads, d), dtype=u8, device=dev),
        "k8": torch.empty((heads, t, L.H3_FP8_QK_BLOCK, d), dtype=u8, device=dev),
        "v8t": torch.empty((heads, t, d, L.H3_FP8_QK_BLOCK), dtype=u8, device=dev),
        "q_scale": torch.empty((t, heads), dtype=torch.float32, device=dev),
        "k_scale": torch.empty((t, heads), dtype=torch.float32, device=dev),
        "v_scale": torch.empty((b, heads, d), dtype=torch.float32, device=dev),
    }
    ws = _workspace(lib().h3_fp8_quantize_workspace_size(b, n, heads), dev, workspace)
    check(lib().h3_fp8_quantize(_ptr(q), _ptr(k), _ptr(v), *strides, _ptr(cu_seqlens),
                                cu.ctypes.data_as(C.c_void_p), b, n, heads, d, _ptr(out["q8"]),
                                _ptr(out["k8"]), _ptr(out["v8t"]), _ptr(out["q_scale"]),
                                _ptr(out["k_scale"]), _ptr(out["v_scale"]), _ptr(ws), ws.numel(),
                                _stream(dev)))
    return out


def attn_block_sparse_list_stride(cu_host, sparsity: float) -> int:
    """Entries per list row of attn_block_sparse's kept-block lists."""
    cu = _host_cu(cu_host)
    stride = C.c_int64(0)
    check(lib().h3_attn_block_sparse_list_stride(cu.ctypes.data_as(C.c_void_p), cu.size - 1,
                                                 float(sparsity), C.byref(stride)))
    return stride.value


def attn_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                      cu_host, sparsity: float = 0.8, softmax_scale: float = 0.0,
                      out: Optional[torch.Tensor] = None, kv_block_lists: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-sparse varlen attention, INT8 Q/K + FP8 V (h3_attn_block_sparse);
    q, k, v, out [N, H, 128] bf16. kv_block_lists, if given, is int32
    [H, T, attn_block_sparse_list_stride(cu_host, sparsity)] and receives
    the kept key blocks of each (head, 256-row query block)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, BF16, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n, heads, d = q.shape
    if out is None:
        out = torch.empty((n, heads, d), dtype=BF16, device=dev)
    _need(out, "out", BF16, dev)
    strides = [_token_view(t, nm, heads, d) for nm, t in (("q", q), ("k", k), ("v", v), ("out", out))]
    cu = _host_cu(cu_host)
    if kv_block_lists is not None:
        _need(kv_block_lists, "kv_block_lists", torch.int32, dev)
        want = (heads, fp8_num_tiles(cu), attn_block_sparse_list_stride(cu, sparsity))
        if tuple(kv_block_lists.shape) != want or not kv_block_lists.is_contiguous():
            raise ValueError(f"kv_block_lists must be a contiguous int32 tensor of shape {want}")
    nbytes = lib().h3_attn_block_sparse_workspace_size(cu.size - 1, n, heads, d, float(sparsity))
    ws = _workspace(nbytes, dev, workspace)
    check(lib().h3_attn_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), *strides, _ptr(cu_seqlens),
                                     cu.ctypes.data_as(C.c_void_p), cu.size - 1, n, heads, d,
                                     float(softmax_scale), float(sparsity),
                                     None if kv_block_lists is None else _ptr(kv_block_lists),
                                     _ptr(ws), ws.numel(), _stream(dev)))
    return out


def dense_attention_step(step: int, num_steps: int, start_steps: int, end_steps: int) -> bool:
    """Whether denoising step `step` (0-based) runs dense attention under the
    block-sparse configuration: the first start_steps and the last end_steps
    of num_steps do (the dense-fallback window, counts not indices)."""
    if not 0 <= step < num_steps or start_steps < 0 or end_steps < 0:
        raise ValueError("step, start_steps or end_steps out of range")
    return step < start_steps or step >= num_steps - end_steps


# --------------------------------------------------------------------------
# Per-block fused operators
# --------------------------------------------------------------------------

def qk_rmsnorm_rope(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                    rope_grid: torch.Tensor, rope_split: Sequence[int], theta: float = 10000.0,
                    eps: float = 1e-6) -> None:
    """In place on q and k ([N, H, D] bf16 views with contiguous heads)."""
    dev = q.device
    _need(q, "q", BF16, dev)
    _need(k, "k", BF16, dev)
    _need(w_q, "w_q", BF16, dev)
    _need(w_k, "w_k", BF16, dev)
    _need(rope_grid, "rope_grid", torch.int32, dev)
    n, heads, d = q.shape
    qs = _token_view(q, "q", heads, d)
    ks = _token_view(k, "k", heads, d)
    if not rope_grid.is_contiguous() or tuple(rope_grid.shape) != (n, 3):
        raise ValueError("rope_grid must be a contiguous [N, 3] int32 tensor")
    if w_q.numel() != d or w_k.numel() != d:
        raise ValueError("gains must have head_dim elements")
    split = (C.c_int32 * 3)(*[int(s) for s in rope_split])
    check(lib().h3_qk_rmsnorm_rope(_ptr(q), _ptr(k), qs, ks, _ptr(w_q.contiguous()),
                                   _ptr(w_k.contiguous()), _ptr(rope_grid), n, heads, d, split,
                                   float(theta), float(eps), _stream(dev)))


def modulation(cond: torch.Tensor, w_mod: torch.Tensor) -> torch.Tensor:
    """fp32 [B, 6C] = cond [B, C] . W_mod^T."""
    dev = cond.device
    _need(cond, "cond", BF16, dev)
    _need(w_mod, "w_mod", BF16, dev)
    b, c = cond.shape
    if tuple(w_mod.shape) != (6 * c, c) or not w_mod.is_contiguous() or not cond.is_contiguous():
        raise ValueError("w_mod must be contiguous [6C, C] and cond contiguous [B, C]")
    mod = torch.empty((b, 6 * c), dtype=torch.float32, device=dev)
    check(lib().h3_modulation(_ptr(cond), _ptr(w_mod), _ptr(mod), b, c, _stream(dev)))
    return mod


def adaln_rmsnorm_modulate(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor,
                           cu_seqlens: torch.Tensor, cu_host, eps: float = 1e-6,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h = RMSNorm(x) * (1 + scale[seg]) + shift[seg]; shift/scale fp32 [B, C] views
    whose rows may be strided (e.g. slices of the modulation output)."""
    dev = x.device
    _need(x, "x", BF16, dev)
    _need(shift, "shift", torch.float32, dev)
    _need(scale, "scale", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n, c = x.shape
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if shift.stride(1) != 1 or scale.stride(1) != 1 or shift.stride(0) != scale.stride(0):
        raise ValueError("shift/scale rows must be contiguous with one common row stride")
    if out is None:
        out = torch.empty_like(x)
    cu = _host_cu(cu_host)
    check(lib().h3_adaln_rmsnorm_modulate(_ptr(x), _ptr(out), _ptr(shift), _ptr(scale),
                                          shift.stride(0), _ptr(cu_seqlens),
                                          cu.ctypes.data_as(C.c_void_p), cu.size - 1, n, c,
                                          float(eps), _stream(dev)))
    return out


def _gemm_args(a, ws, name="w"):
    dev = a.device
    _need(a, "a", BF16, dev)
    for i, w in enumerate(ws):
        _need(w, f"{name}{i}", BF16, dev)
        if not w.is_contiguous():
            raise ValueError("weights must be contiguous")
    if not a.is_contiguous():
        raise ValueError("a must be contiguous")
    return dev


def linear(a: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    dev = _gemm_args(a, [w])
    m, k = a.shape
    n = w.shape[0]
    y = torch.empty((m, n), dtype=BF16, device=dev)
    check(lib().h3_linear_bf16(_ptr(a), _ptr(w), _ptr(y), m, n, k, _stream(dev)))
    return y


def linear_swiglu(a: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    dev = _gemm_args(a, [w_gate, w_up])
    m, k = a.shape
    n = w_gate.shape[0]
    if tuple(w_up.shape) != tuple(w_gate.shape):
        raise ValueError("w_gate and w_up must have the same shape")
    y = torch.empty((m, n), dtype=BF16, device=dev)
    check(lib().h3_linear_swiglu_bf16(_ptr(a), _ptr(w_gate), _ptr(w_up), _ptr(y), m, n, k,
                                      _stream(dev)))
    return y


def linear_gated_residual(a: torch.Tensor, w: torch.Tensor, res: torch.Tensor,
                          gate: torch.Tensor, cu_seqlens: torch.Tensor, cu_host,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dev = _gemm_args(a, [w])
    _need(res, "res", BF16, dev)
    _need(gate, "gate", torch.float32, dev)
    m, k = a.shape
    n = w.shape[0]
    if gate.stride(1) != 1:
        raise ValueError("gate rows must be contiguous")
    y = torch.empty((m, n), dtype=BF16, device=dev) if out is None else out
    cu = _host_cu(cu_host)
    check(lib().h3_linear_gated_residual_bf16(_ptr(a), _ptr(w), _ptr(res.contiguous()),
                                              _ptr(gate), gate.stride(0), _ptr(y), m, n, k,
                                              _ptr(cu_seqlens), cu.ctypes.data_as(C.c_void_p),
                                              cu.size - 1, _stream(dev)))
    return y


def frames_to_uint8_bthwc(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 decoded frames [B, C, T, H, W] -> uint8 [B, T, H, W, C]."""
    _need(x, "x", torch.float32)
    if x.dim() != 5 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, C, T, H, W] tensor")
    b, c, t, h, w = x.shape
    if out is None:
        out = torch.empty((b, t, h, w, c), dtype=torch.uint8, device=x.device)
    if out.dtype != torch.uint8 or tuple(out.shape) != (b, t, h, w, c) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 [B, T, H, W, C] tensor")
    check(lib().h3_frames_to_uint8_bthwc(_ptr(x), _ptr(out), b, c, t, h, w, _stream(x.device)))
    return out


# --------------------------------------------------------------------------
# MXFP8 (layouts in h3dit.h: codes [rows, k] uint8, scales K-step-major)
# --------------------------------------------------------------------------

class MX:
    """An MXFP8 matrix: `codes` uint8 [rows, k] (E4M3) and `scales` uint8
    [rows * k / 32] (E8M0, K-step-major)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or codes.dim() != 2:
            raise TypeError("MX codes must be uint8 [rows, k] and scales uint8")
        rows, k = codes.shape
        if k % 128 or scales.numel() != rows * k // 32 or not codes.is_contiguous():
            raise ValueError("MX: k must be a multiple of 128, codes contiguous, scales rows*k/32 bytes")
        self.codes, self.scales = codes, scales

    @property
    def shape(self):
        return tuple(self.codes.shape)

    @staticmethod
    def empty(rows: int, k: int, device) -> "MX":
        return MX(torch.empty((rows, k), dtype=torch.uint8, device=device),
                  torch.empty(rows * k // 32, dtype=torch.uint8, device=device))


def mx_quantize(x: torch.Tensor, out: Optional[MX] = None) -> MX:
    """MXFP8 codes and scales of bf16 x [rows, k] (rows may be strided)."""
    _need(x, "x", BF16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [rows, k] with contiguous rows")
    rows, k = x.shape
    out = MX.empty(rows, k, x.device) if out is None else out
    if out.shape != (rows, k):
        raise ValueError("out has the wrong shape")
    check(lib().h3_mx_quantize_bf16(_ptr(x), x.stride(0), rows, k, _ptr(out.codes), _ptr(out.scales),
                                    _stream(x.device)))
    return out


def adaln_rmsnorm_modulate_mx(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor,
                              cu_seqlens: torch.Tensor, cu_host, eps: float = 1e-6,
                              out: Optional[MX] = None) -> MX:
    """MX(RMSNorm(x) * (1 + scale[seg]) + shift[seg]), quantised from fp32."""
    dev = x.device
    _need(x, "x", BF16, dev)
    _need(shift, "shift", torch.float32, dev)
    _need(scale, "scale", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n, c = x.shape
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if shift.stride(1) != 1 or scale.stride(1) != 1 or shift.stride(0) != scale.stride(0):
        raise ValueError("shift/scale rows must be contiguous with one common row stride")
    out = MX.empty(n, c, dev) if out is None else out
    cu = _host_cu(cu_host)
    check(lib().h3_adaln_rmsnorm_modulate_mxfp8(_ptr(x), _ptr(out.codes), _ptr(out.scales), _ptr(shift),
                                                _ptr(scale), shift.stride(0), _ptr(cu_seqlens),
                                                cu.ctypes.data_as(C.c_void_p), cu.size - 1, n, c,
                                                float(eps), _stream(dev)))
    return out


def _mx_args(a: MX, ws) -> torch.device:
    dev = a.codes.device
    for t in [a] + list(ws):
        if not isinstance(t, MX):
            raise TypeError("MX operands expected")
        if t.codes.device != dev:
            raise ValueError("operands on different devices")
        if t.shape[1] != a.shape[1]:
            raise ValueError("operands must share k")
    return dev


def linear_mx(a: MX, w: MX) -> torch.Tensor:
    """y = dq(a) dq(w)^T in bf16."""
    dev = _mx_args(a, [w])
    m, k = a.shape
    n = w.shape[0]
    y = torch.empty((m, n), dtype=BF16, device=dev)
    check(lib().h3_linear_mxfp8(_ptr(a.codes), _ptr(a.scales), _ptr(w.codes), _ptr(w.scales), _ptr(y),
                                m, n, k, _stream(dev)))
    return y


def linear_swiglu_mx(a: MX, w_gate: MX, w_up: MX, out: Optional[MX] = None) -> MX:
    """MX(silu(dq(a) dq(w_gate)^T) * (dq(a) dq(w_up)^T))."""
    dev = _mx_args(a, [w_gate, w_up])
    m, k = a.shape
    n = w_gate.shape[0]
    if w_up.shape != w_gate.shape:
        raise ValueError("w_gate and w_up must have the same shape")
    y = MX.empty(m, n, dev) if out is None else out
    check(lib().h3_linear_swiglu_mxfp8(_ptr(a.codes), _ptr(a.scales), _ptr(w_gate.codes),
                                       _ptr(w_gate.scales), _ptr(w_up.codes), _ptr(w_up.scales),
                                       _ptr(y.codes), _ptr(y.scales), m, n, k, _stream(dev)))
    return y


def linear_gated_residual_mx(a: MX, w: MX, res: torch.Tensor, gate: torch.Tensor,
                             cu_seqlens: torch.Tensor, cu_host,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dev = _mx_args(a, [w])
    _need(res, "res", BF16, dev)
    _need(gate, "gate", torch.float32, dev)
    m, k = a.shape
    n = w.shape[0]
    if gate.stride(1) != 1:
        raise ValueError("gate rows must be contiguous")
    y = torch.empty((m, n), dtype=BF16, device=dev) if out is None else out
    cu = _host_cu(cu_host)
    check(lib().h3_linear_gated_residual_mxfp8(_ptr(a.codes), _ptr(a.scales), _ptr(w.codes),
                                               _ptr(w.scales), _ptr(res.contiguous()), _ptr(gate),
                                               gate.stride(0), _ptr(y), m, n, k, _ptr(cu_seqlens),
                                               cu.ctypes.data_as(C.c_void_p), cu.size - 1,
                                               _stream(dev)))
    return y


# --------------------------------------------------------------------------
# The block
# --------------------------------------------------------------------------

WEIGHT_NAMES = ("w_mod", "w_qkv", "w_o", "q_norm", "k_norm", "w_gate", "w_up", "w_down")
TAP_NAMES = ("mod", "h", "qkv", "o", "x1", "h2", "a")


class DitBlock:
    """One block's dims and device weights; forward() calls h3_dit_block_forward."""

    def __init__(self, weights: Dict[str, torch.Tensor], heads: int, head_dim: int,
                 ffn_dim: int, rope_split: Sequence[int], rope_theta: float = 10000.0,
                 eps: float = 1e-6):
        self.weights = weights
        hidden = heads * head_dim
        for nm in WEIGHT_NAMES:
            _need(weights[nm], nm, BF16)
            if not weights[nm].is_contiguous():
                raise ValueError(f"{nm} must be contiguous")
        self.dims = DitDims(hidden, heads, head_dim, ffn_dim, (C.c_int32 * 3)(*rope_split),
                            float(rope_theta), float(eps))
        self.c_weights = DitWeights(*[weights[nm].data_ptr() for nm in WEIGHT_NAMES])
        self.hidden, self.ffn = hidden, ffn_dim

    def workspace_bytes(self, num_seqs: int, total_tokens: int) -> int:
        return lib().h3_dit_block_workspace_size(C.byref(self.dims), num_seqs, total_tokens)

    def forward(self, x: torch.Tensor, cond: torch.Tensor, cu_seqlens: torch.Tensor, cu_host,
                rope_grid: torch.Tensor, out: Optional[torch.Tensor] = None,
                taps: Optional[Dict[str, torch.Tensor]] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        dev = x.device
        _need(x, "x", BF16, dev)
        _need(cond, "cond", BF16, dev)
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        _need(rope_grid, "rope_grid", torch.int32, dev)
        if not (x.is_contiguous() and cond.is_contiguous() and rope_grid.is_contiguous()):
            raise ValueError("x, cond and rope_grid must be contiguous")
        cu = _host_cu(cu_host)
        b, n = cu.size - 1, x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        ws = _workspace(self.workspace_bytes(b, n), dev, workspace)
        c_taps = None
        if taps is not None:
            c_taps = DitTaps(*[None if taps.get(nm) is None else taps[nm].data_ptr()
                               for nm in TAP_NAMES])
        check(lib().h3_dit_block_forward(_ptr(x), _ptr(out), _ptr(cond), C.byref(self.c_weights),
                                         C.byref(self.dims), _ptr(cu_seqlens),
                                         cu.ctypes.data_as(C.c_void_p), b, n, _ptr(rope_grid),
                                         None if c_taps is None else C.byref(c_taps), _ptr(ws),
                                         ws.numel(), _stream(dev)))
        return out

    def make_taps(self, num_seqs: int, total_tokens: int, device) -> Dict[str, torch.Tensor]:
        n, c = total_tokens, self.hidden
        return {"mod": torch.empty((num_seqs, 6 * c), dtype=torch.float32, device=device),
                "h": torch.empty((n, c), dtype=BF16, device=device),
                "qkv": torch.empty((n, 3 * c), dtype=BF16, device=device),
                "o": torch.empty((n, c), dtype=BF16, device=device),
                "x1": torch.empty((n, c), dtype=BF16, device=device),
                "h2": torch.empty((n, c), dtype=BF16, device=device),
                "a": torch.empty((n, self.ffn), dtype=BF16, device=device)}


MX_WEIGHT_NAMES = ("w_qkv", "w_o", "w_gate", "w_up", "w_down")


class DitBlockMX:
    """The block with MXFP8 linears: the five linear weights are quantised
    once here (h3_mx_quantize_bf16); forward() calls h3_dit_block_forward_mxfp8,
    or, with attn_sparsity set, h3_dit_block_forward_mxfp8_bsa (block-sparse
    INT8/FP8 attention at that sparsity: the pages' lossy configuration)."""

    def __init__(self, weights: Dict[str, torch.Tensor], heads: int, head_dim: int,
                 ffn_dim: int, rope_split: Sequence[int], rope_theta: float = 10000.0,
                 eps: float = 1e-6, attn_sparsity: Optional[float] = None):
        self.attn_sparsity = None if attn_sparsity is None else float(attn_sparsity)
        hidden = heads * head_dim
        for nm in WEIGHT_NAMES:
            _need(weights[nm], nm, BF16)
            if not weights[nm].is_contiguous():
                raise ValueError(f"{nm} must be contiguous")
        self.bf16 = {nm: weights[nm] for nm in ("w_mod", "q_norm", "k_norm")}
        self.mx = {nm: mx_quantize(weights[nm]) for nm in MX_WEIGHT_NAMES}
        self.dims = DitDims(hidden, heads, head_dim, ffn_dim, (C.c_int32 * 3)(*rope_split),
                            float(rope_theta), float(eps))
        mats = [MxMatrix(self.mx[nm].codes.data_ptr(), self.mx[nm].scales.data_ptr())
                for nm in MX_WEIGHT_NAMES]
        self.c_weights = DitMxWeights(self.bf16["w_mod"].data_ptr(), self.bf16["q_norm"].data_ptr(),
                                      self.bf16["k_norm"].data_ptr(), *mats)
        self.hidden, self.ffn = hidden, ffn_dim

    def workspace_bytes(self, num_seqs: int, total_tokens: int) -> int:
        if self.attn_sparsity is not None:
            return lib().h3_dit_block_mx_bsa_workspace_size(C.byref(self.dims), num_seqs, total_tokens,
                                                            self.attn_sparsity)
        return lib().h3_dit_block_mx_workspace_size(C.byref(self.dims), num_seqs, total_tokens)

    def forward(self, x: torch.Tensor, cond: torch.Tensor, cu_seqlens: torch.Tensor, cu_host,
                rope_grid: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        dev = x.device
        _need(x, "x", BF16, dev)
        _need(cond, "cond", BF16, dev)
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        _need(rope_grid, "rope_grid", torch.int32, dev)
        if not (x.is_contiguous() and cond.is_contiguous() and rope_grid.is_contiguous()):
            raise ValueError("x, cond and rope_grid must be contiguous")
        cu = _host_cu(cu_host)
        b, n = cu.size - 1, x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        ws = _workspace(self.workspace_bytes(b, n), dev, workspace)
        common = (_ptr(x), _ptr(out), _ptr(cond), C.byref(self.c_weights), C.byref(self.dims),
                  _ptr(cu_seqlens), cu.ctypes.data_as(C.c_void_p), b, n, _ptr(rope_grid))
        if self.attn_sparsity is not None:
            check(lib().h3_dit_block_forward_mxfp8_bsa(*common, self.attn_sparsity, _ptr(ws), ws.numel(),
                                                       _stream(dev)))
        else:
            check(lib().h3_dit_block_forward_mxfp8(*common, _ptr(ws), ws.numel(), _stream(dev)))
        return out


# --------------------------------------------------------------------------
# MXFP4 linears and the block with them
# --------------------------------------------------------------------------

class MX4:
    """An MXFP4 matrix [rows, k]: `codes` uint8 [rows, k / 2] (two E2M1
    codes per byte, element 2i in the low nibble) and `scales` uint8
    [rows * k / 32] (E8M0, 8 bytes per row and 256-element K step)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, k: int):
        if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or codes.dim() != 2:
            raise TypeError("MX4 codes must be uint8 [rows, k / 2] and scales uint8")
        rows = codes.shape[0]
        if k % 256 or codes.shape[1] * 2 != k or scales.numel() != rows * k // 32 or not codes.is_contiguous():
            raise ValueError("MX4: k must be a multiple of 256, codes contiguous [rows, k/2], scales rows*k/32")
        self.codes, self.scales, self.k = codes, scales, k

    @property
    def shape(self):
        return (self.codes.shape[0], self.k)

    @staticmethod
    def empty(rows: int, k: int, device) -> "MX4":
        return MX4(torch.empty((rows, k // 2), dtype=torch.uint8, device=device),
                   torch.empty(rows * k // 32, dtype=torch.uint8, device=device), k)


def mx4_quantize(x: torch.Tensor, out: Optional[MX4] = None) -> MX4:
    """MXFP4 codes and scales of bf16 x [rows, k] (rows may be strided)."""
    _need(x, "x", BF16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [rows, k] with contiguous rows")
    rows, k = x.shape
    out = MX4.empty(rows, k, x.device) if out is None else out
    if out.shape != (rows, k):
        raise ValueError("out has the wrong shape")
    check(lib().h3_mx4_quantize_bf16(_ptr(x), x.stride(0), rows, k, _ptr(out.codes), _ptr(out.scales),
                                     _stream(x.device)))
    return out


def _mx4_args(a: MX4, ws) -> torch.device:
    dev = a.codes.device
    for t in [a] + list(ws):
        if not isinstance(t, MX4):
            raise TypeError("MX4 operands expected")
        if t.codes.device != dev:
            raise ValueError("operands on different devices")
        if t.shape[1] != a.shape[1]:
            raise ValueError("operands must share k")
    return dev


def linear_mx4(a: MX4, w: MX4, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = dq(a) dq(w)^T in bf16 (MXFP4 operands)."""
    dev = _mx4_args(a, [w])
    m, k = a.shape
    n = w.shape[0]
    y = torch.empty((m, n), dtype=BF16, device=dev) if out is None else out
    check(lib().h3_linear_mxfp4(_ptr(a.codes), _ptr(a.scales), _ptr(w.codes), _ptr(w.scales), _ptr(y),
                                m, n, k, _stream(dev)))
    return y


def linear_swiglu_mx4(a: MX4, w_gate: MX4, w_up: MX4, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """silu(dq(a) dq(w_gate)^T) * (dq(a) dq(w_up)^T) in bf16 (MXFP4 operands)."""
    dev = _mx4_args(a, [w_gate, w_up])
    m, k = a.shape
    n = w_gate.shape[0]
    if w_up.shape != w_gate.shape:
        raise ValueError("w_gate and w_up must have the same shape")
    y = torch.empty((m, n), dtype=BF16, device=dev) if out is None else out
    check(lib().h3_linear_swiglu_mxfp4(_ptr(a.codes), _ptr(a.scales), _ptr(w_gate.codes),
                                       _ptr(w_gate.scales), _ptr(w_up.codes), _ptr(w_up.scales),
                                       _ptr(y), m, n, k, _stream(dev)))
    return y


def linear_gated_residual_mx4(a: MX4, w: MX4, res: torch.Tensor, gate: torch.Tensor,
                              cu_seqlens: torch.Tensor, cu_host,
                              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dev = _mx4_args(a, [w])
    _need(res, "res", BF16, dev)
    _need(gate, "gate", torch.float32, dev)
    m, k = a.shape
    n = w.shape[0]
    if gate.stride(1) != 1:
        raise ValueError("gate rows must be contiguous")
    y = torch.empty((m, n), dtype=BF16, device=dev) if out is None else out
    cu = _host_cu(cu_host)
    check(lib().h3_linear_gated_residual_mxfp4(_ptr(a.codes), _ptr(a.scales), _ptr(w.codes),
                                               _ptr(w.scales), _ptr(res.contiguous()), _ptr(gate),
                                               gate.stride(0), _ptr(y), m, n, k, _ptr(cu_seqlens),
                                               cu.ctypes.data_as(C.c_void_p), cu.size - 1,
                                               _stream(dev)))
    return y


class DitBlockMX4:
    """The block with MXFP4 linears: the five linear weights are quantised
    once here (h3_mx4_quantize_bf16); forward() calls h3_dit_block_forward_mxfp4."""

    def __init__(self, weights: Dict[str, torch.Tensor], heads: int, head_dim: int,
                 ffn_dim: int, rope_split: Sequence[int], rope_theta: float = 10000.0,
                 eps: float = 1e-6):
        hidden = heads * head_dim
        for nm in WEIGHT_NAMES:
            _need(weights[nm], nm, BF16)
            if not weights[nm].is_contiguous():
                raise ValueError(f"{nm} must be contiguous")
        self.bf16 = {nm: weights[nm] for nm in ("w_mod", "q_norm", "k_norm")}
        self.mx = {nm: mx4_quantize(weights[nm]) for nm in MX_WEIGHT_NAMES}
        self.dims = DitDims(hidden, heads, head_dim, ffn_dim, (C.c_int32 * 3)(*rope_split),
                            float(rope_theta), float(eps))
        mats = [MxMatrix(self.mx[nm].codes.data_ptr(), self.mx[nm].scales.data_ptr())
                for nm in MX_WEIGHT_NAMES]
        self.c_weights = DitMxWeights(self.bf16["w_mod"].data_ptr(), self.bf16["q_norm"].data_ptr(),
                                      self.bf16["k_norm"].data_ptr(), *mats)
        self.hidden, self.ffn = hidden, ffn_dim

    def workspace_bytes(self, num_seqs: int, total_tokens: int) -> int:
        return lib().h3_dit_block_mx4_workspace_size(C.byref(self.dims), num_seqs, total_tokens)

    def forward(self, x: torch.Tensor, cond: torch.Tensor, cu_seqlens: torch.Tensor, cu_host,
                rope_grid: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        dev = x.device
        _need(x, "x", BF16, dev)
        _need(cond, "cond", BF16, dev)
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        _need(rope_grid, "rope_grid", torch.int32, dev)
        if not (x.is_contiguous() and cond.is_contiguous() and rope_grid.is_contiguous()):
            raise ValueError("x, cond and rope_grid must be contiguous")
        cu = _host_cu(cu_host)
        b, n = cu.size - 1, x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        ws = _workspace(self.workspace_bytes(b, n), dev, workspace)
        check(lib().h3_dit_block_forward_mxfp4(_ptr(x), _ptr(out), _ptr(cond), C.byref(self.c_weights),
                                               C.byref(self.dims), _ptr(cu_seqlens),
                                               cu.ctypes.data_as(C.c_void_p), b, n, _ptr(rope_grid),
                                               _ptr(ws), ws.numel(), _stream(dev)))
        return out
