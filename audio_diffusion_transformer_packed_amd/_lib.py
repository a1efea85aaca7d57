"""ctypes loader and signatures of libh3dit.so (the C ABI of include/h3dit.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any operation.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libh3dit.so")

H3_OK = 0
H3_ERR_INVALID_ARGUMENT = 1
H3_ERR_UNSUPPORTED = 2
H3_ERR_WORKSPACE_TOO_SMALL = 3
H3_ERR_HIP = 4

H3_ATTN_BF16 = 0
H3_ATTN_FP8_E4M3 = 1
H3_ATTN_BLOCK_M = 256
H3_FP8_QK_BLOCK = 64

# Every exported symbol, in header order.
EXPORTS = (
    "h3_status_string", "h3_last_error_message", "h3_abi_version", "h3_build_schedule_host",
    "h3_varlen_bookkeeping_workspace_size", "h3_varlen_bookkeeping",
    "h3_attn_varlen_workspace_size", "h3_attn_varlen_num_items", "h3_attn_varlen",
    "h3_attn_varlen_noalloc",
    "h3_fp8_num_tiles", "h3_fp8_quantize_workspace_size", "h3_fp8_quantize",
    "h3_attn_block_sparse_list_stride", "h3_attn_block_sparse_workspace_size",
    "h3_attn_block_sparse", "h3_qk_rmsnorm_rope", "h3_modulation", "h3_adaln_rmsnorm_modulate", "h3_linear_bf16",
    "h3_linear_swiglu_bf16", "h3_linear_gated_residual_bf16", "h3_frames_to_uint8_bthwc",
    "h3_adaln_rmsnorm_modulate_mxfp8",
    "h3_mx_quantize_bf16",
    "h3_linear_mxfp8", "h3_linear_swiglu_mxfp8", "h3_linear_gated_residual_mxfp8",
    "h3_dit_block_workspace_size", "h3_dit_block_forward", "h3_dit_block_mx_workspace_size",
    "h3_dit_block_forward_mxfp8", "h3_dit_block_mx_bsa_workspace_size", "h3_dit_block_forward_mxfp8_bsa",
    "h3_mx4_quantize_bf16", "h3_linear_mxfp4", "h3_linear_swiglu_mxfp4", "h3_linear_gated_residual_mxfp4",
    "h3_dit_block_mx4_workspace_size", "h3_dit_block_forward_mxfp4",
)


class AttnOpts(C.Structure):
    _fields_ = [("precision", C.c_int32), ("skip_softmax", C.c_int32),
                ("skip_threshold", C.c_float), ("softmax_scale", C.c_float),
                ("skip_counts", C.c_void_p)]


class DitDims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn_dim", C.c_int32), ("rope_split", C.c_int32 * 3),
                ("rope_theta", C.c_float), ("eps", C.c_float)]


class DitWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("w_mod", "w_qkv", "w_o", "q_norm", "k_norm", "w_gate", "w_up", "w_down")]


class MxMatrix(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p)]


class DitMxWeights(C.Structure):
    _fields_ = [("w_mod", C.c_void_p), ("q_norm", C.c_void_p), ("k_norm", C.c_void_p)] + \
               [(n, MxMatrix) for n in ("w_qkv", "w_o", "w_gate", "w_up", "w_down")]


class DitTaps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("mod", "h", "qkv", "o", "x1", "h2", "a")]


class H3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_lib = None
P = C.c_void_p
I32, I64, F32, SZ = C.c_int32, C.c_int64, C.c_float, C.c_size_t


def _declare(lib):
    sig = {
        "h3_status_string": (C.c_char_p, [C.c_int]),
        "h3_last_error_message": (C.c_char_p, []),
        "h3_abi_version": (I32, []),
        "h3_build_schedule_host": (C.c_int, [P, I32, I32, I32, P, I64, P]),
        "h3_varlen_bookkeeping_workspace_size": (SZ, [I32]),
        "h3_varlen_bookkeeping": (C.c_int, [P, P, I32, I32, I32, I32, P, P, P, I64, P, SZ, P]),
        "h3_attn_varlen_workspace_size": (SZ, [I32, I32, I32, I32, P]),
        "h3_attn_varlen_num_items": (C.c_int, [P, I32, I32, P]),
        "h3_attn_varlen": (C.c_int, [P, P, P, P, I64, I64, I64, I64, P, P, I32, I32, I32, I32, P,
                                     P, SZ, P]),
        "h3_attn_varlen_noalloc": (C.c_int, [P, P, P, P, I64, I64, I64, I64, P, P, I32, I32, I32,
                                             I32, P, P]),
        "h3_fp8_num_tiles": (C.c_int, [P, I32, P]),
        "h3_fp8_quantize_workspace_size": (SZ, [I32, I32, I32]),
        "h3_fp8_quantize": (C.c_int, [P, P, P, I64, I64, I64, P, P, I32, I32, I32, I32, P, P, P, P,
                                      P, P, P, SZ, P]),
        "h3_attn_block_sparse_list_stride": (C.c_int, [P, I32, F32, P]),
        "h3_attn_block_sparse_workspace_size": (SZ, [I32, I32, I32, I32, F32]),
        "h3_attn_block_sparse": (C.c_int, [P, P, P, P, I64, I64, I64, I64, P, P, I32, I32, I32, I32,
                                           F32, F32, P, P, SZ, P]),
        "h3_qk_rmsnorm_rope": (C.c_int, [P, P, I64, I64, P, P, P, I32, I32, I32, P, F32, F32, P]),
        "h3_modulation": (C.c_int, [P, P, P, I32, I32, P]),
        "h3_adaln_rmsnorm_modulate": (C.c_int, [P, P, P, P, I64, P, P, I32, I32, I32, F32, P]),
        "h3_linear_bf16": (C.c_int, [P, P, P, I64, I64, I64, P]),
        "h3_linear_swiglu_bf16": (C.c_int, [P, P, P, P, I64, I64, I64, P]),
        "h3_linear_gated_residual_bf16": (C.c_int, [P, P, P, P, I64, P, I64, I64, I64, P, P, I32,
                                                    P]),
        "h3_frames_to_uint8_bthwc": (C.c_int, [P, P, I64, I64, I64, I64, I64, P]),
        "h3_adaln_rmsnorm_modulate_mxfp8": (C.c_int, [P, P, P, P, P, I64, P, P, I32, I32, I32, F32,
                                                      P]),
        "h3_mx4_quantize_bf16": (C.c_int, [P, I64, I64, I64, P, P, P]),
        "h3_linear_mxfp4": (C.c_int, [P, P, P, P, P, I64, I64, I64, P]),
        "h3_linear_swiglu_mxfp4": (C.c_int, [P, P, P, P, P, P, P, I64, I64, I64, P]),
        "h3_linear_gated_residual_mxfp4": (C.c_int, [P, P, P, P, P, P, I64, P, I64, I64, I64, P, P, I32,
                                                     P]),
        "h3_dit_block_mx4_workspace_size": (SZ, [P, I32, I32]),
        "h3_dit_block_forward_mxfp4": (C.c_int, [P, P, P, P, P, P, P, I32, I32, P, P, SZ, P]),
        "h3_mx_quantize_bf16": (C.c_int, [P, I64, I64, I64, P, P, P]),
        "h3_linear_mxfp8": (C.c_int, [P, P, P, P, P, I64, I64, I64, P]),
        "h3_linear_swiglu_mxfp8": (C.c_int, [P, P, P, P, P, P, P, P, I64, I64, I64, P]),
        "h3_linear_gated_residual_mxfp8": (C.c_int, [P, P, P, P, P, P, I64, P, I64, I64, I64, P, P,
                                                     I32, P]),
        "h3_dit_block_workspace_size": (SZ, [P, I32, I32]),
        "h3_dit_block_forward": (C.c_int, [P, P, P, P, P, P, P, I32, I32, P, P, P, SZ, P]),
        "h3_dit_block_mx_workspace_size": (SZ, [P, I32, I32]),
        "h3_dit_block_forward_mxfp8": (C.c_int, [P, P, P, P, P, P, P, I32, I32, P, P, SZ, P]),
        "h3_dit_block_mx_bsa_workspace_size": (SZ, [P, I32, I32, F32]),
        "h3_dit_block_forward_mxfp8_bsa": (C.c_int, [P, P, P, P, P, P, P, I32, I32, P, F32, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m audio_diffusion_transformer_packed_amd.build)")
        handle = C.CDLL(LIB_PATH)
        _declare(handle)
        _lib = handle
    return _lib


def status_name(status: int) -> str:
    try:
        return lib().h3_status_string(status).decode()
    except Exception:  # the library itself may be what failed to load
        return f"status {status}"


def check(status: int) -> None:
    if status != H3_OK:
        raise H3Error(status, lib().h3_last_error_message().decode())
