"""Helpers shared by the GPU parity tests: device transfer of the seeded
inputs and the bf16 comparison bar."""
from __future__ import annotations

import sys

import numpy as np
import pytest

REL_FRO_BF16 = 1e-2     # relative Frobenius error, bf16 paths
SCALED_ABS_BF16 = 2e-2  # |gpu - ref| <= 2e-2 * max(1, |ref|), bf16 paths


def torch_device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def to_dev_bf16(arr, device):
    """Bf16Array (or uint16 bits) -> device bfloat16 tensor with those exact bits."""
    import torch
    bits = arr.bits if hasattr(arr, "bits") else arr
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def to_dev_i32(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits_of(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def compare(got, ref, name: str, rel_fro: float = REL_FRO_BF16,
            scaled_abs: float = SCALED_ABS_BF16, mag=None):
    """Assert the bf16 bar; print the figures (relF, scaled and literal max-abs).

    Elementwise: |got - ref| <= scaled_abs * max(1, mag), mag = |ref| unless
    given. For a residual output x + g*y the caller passes mag = |x| + |g*y|:
    the error of a sum scales with the magnitudes of its terms, and the gate
    multiplies the bf16 rounding of the branch it scales.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    diff = np.abs(got - ref)
    den = np.linalg.norm(ref.ravel())
    rel = float(np.linalg.norm(diff.ravel()) / den) if den > 0 else float(np.max(diff, initial=0))
    mag = np.abs(ref) if mag is None else np.asarray(mag, dtype=np.float64)
    scaled = float(np.max(diff / np.maximum(1.0, mag), initial=0.0))
    maxabs = float(np.max(diff, initial=0.0))
    print(f"[parity] {name}: relF={rel:.3e} scaled_max={scaled:.3e} max_abs={maxabs:.3e} "
          f"ref_rms={float(np.sqrt(np.mean(ref * ref))) if ref.size else 0:.3e}")
    sys.stdout.flush()
    assert rel <= rel_fro, f"{name}: relative Frobenius error {rel:.3e} > {rel_fro}"
    assert scaled <= scaled_abs, f"{name}: scaled max error {scaled:.3e} > {scaled_abs}"
    return rel, scaled, maxabs


def announce(msg: str):
    print(f"[gpu-case] {msg}")
    sys.stdout.flush()
