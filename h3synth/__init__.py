"""Seeded synthetic inputs for the packed joint audio-video DiT hot path.

This module is shared by the tests, the bench and the smoke check. It holds
none of the method's arithmetic: it draws random numbers in a fixed order,
rounds them to bf16 and lays out the packed-sequence structure (segment
lengths and the 3D (t, h, w) position of every token). Both the HIP path and
the float64 oracle consume what it returns; neither is imported here.

Workload shapes follow the packed sequences the pages describe (text, audio
and video tokens of one request in one row, about 58k tokens for a 10 s
1344x768 clip; "MiniMax H3 FastH3 real-time serving with vLLM-Omni",
section "System-wide optimizations in vLLM-Omni"). Video latents use a
24 x 42 grid per frame (768/32 x 1344/32).

Every array is produced with numpy's PCG64 generator seeded per workload.
Floating-point draws are float32 standard normals, scaled in float32 where a
standard deviation other than 1 is asked for, then rounded to bf16 with
round-to-nearest-even on the float32 bit pattern. Each array is returned
twice: as float32 values (exactly representable in bf16) and as the raw
uint16 bf16 bit pattern that the device consumes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np

# Seed of the request measured on the pages (serving-configuration section of
# the FastH3 page); each workload adds its own index.
BASE_SEED = 1101

VIDEO_ROWS = 24   # 768 / 32
VIDEO_COLS = 42   # 1344 / 32


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (RNE, NaN-free inputs) and return the uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bits to the float32 values they encode."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Bf16Array:
    """One bf16 tensor: its bits (device input) and its exact float32 value."""
    bits: np.ndarray
    f32: np.ndarray

    @staticmethod
    def from_f32(a: np.ndarray) -> "Bf16Array":
        bits = bf16_bits(a)
        return Bf16Array(bits=bits, f32=bits_to_f32(bits))

    @property
    def shape(self):
        return self.f32.shape


@dataclass
class Request:
    """Token counts of one packed request: text, audio, then a video grid."""
    text: int
    audio: int
    frames: int
    rows: int = VIDEO_ROWS
    cols: int = VIDEO_COLS

    @property
    def video(self) -> int:
        return self.frames * self.rows * self.cols

    @property
    def length(self) -> int:
        return self.text + self.audio + self.video

    def grid(self) -> np.ndarray:
        """(t, h, w) positions: text j -> (j,0,0), audio i -> (i,0,0),
        video (f, r, c) in frame-major raster order -> (f, r, c)."""
        g = np.zeros((self.length, 3), dtype=np.int32)
        g[: self.text, 0] = np.arange(self.text)
        a0 = self.text
        g[a0: a0 + self.audio, 0] = np.arange(self.audio)
        v0 = a0 + self.audio
        f, r, c = np.meshgrid(np.arange(self.frames), np.arange(self.rows),
                              np.arange(self.cols), indexing="ij")
        g[v0:, 0] = f.reshape(-1)
        g[v0:, 1] = r.reshape(-1)
        g[v0:, 2] = c.reshape(-1)
        return g


def pack(requests: Sequence[Request]) -> Tuple[np.ndarray, np.ndarray]:
    """cu_seqlens (int32[B+1]) and the packed position grid (int32[N, 3])."""
    lens = [r.length for r in requests]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    grid = (np.concatenate([r.grid() for r in requests], axis=0)
            if requests else np.zeros((0, 3), np.int32))
    return cu, grid


def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def rope_split_for(head_dim: int) -> Tuple[int, int, int]:
    """(t, h, w) RoPE split: 16/24/24 at head_dim 64 and the same 1:1.5:1.5
    ratio (32/48/48) at head_dim 128."""
    if head_dim == 64:
        return (16, 24, 24)
    if head_dim == 128:
        return (32, 48, 48)
    raise ValueError(f"no RoPE split defined for head_dim {head_dim}")


# --------------------------------------------------------------------------
# Workload definitions
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    index: int
    requests: List[Request]
    heads: int
    head_dim: int
    hidden: int = 0
    ffn: int = 0
    kind: str = "attention"      # "attention" | "block"
    description: str = ""

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def cu_seqlens(self) -> np.ndarray:
        return pack(self.requests)[0]

    @property
    def total_tokens(self) -> int:
        return int(sum(r.length for r in self.requests))

    @property
    def lengths(self) -> List[int]:
        return [r.length for r in self.requests]


WORKLOADS: Dict[str, Workload] = {
    "tiny_packed_2req": Workload(
        name="tiny_packed_2req", index=0,
        requests=[Request(64, 128, 8, 8, 8), Request(64, 128, 5, 8, 8)],
        heads=4, head_dim=64, kind="attention",
        description="two requests packed, cu=[0,704,1216], 4 heads x 64"),
    "attn_5s_32k": Workload(
        name="attn_5s_32k", index=1,
        requests=[Request(512, 500, 31)], heads=24, head_dim=128, kind="attention",
        description="one request of 32,260 tokens (5 s clip), 24 heads x 128"),
    "block_10s_58k": Workload(
        name="block_10s_58k", index=2,
        requests=[Request(512, 1000, 56)], heads=24, head_dim=128,
        hidden=3072, ffn=8192, kind="block",
        description="DiT block over 57,960 packed tokens (10 s clip)"),
    "block_15s_94k": Workload(
        name="block_15s_94k", index=3,
        requests=[Request(512, 1500, 91)], heads=24, head_dim=128,
        hidden=3072, ffn=8192, kind="block",
        description="DiT block over 93,740 packed tokens (15 s clip)"),
    "attn_fp8_10s_58k": Workload(
        name="attn_fp8_10s_58k", index=4,
        requests=[Request(512, 1000, 56)], heads=24, head_dim=128, kind="attention",
        description="fp8 attention at the 10 s shape, 57,960 tokens"),
}


# --------------------------------------------------------------------------
# Generators (fixed draw order per function)
# --------------------------------------------------------------------------

def _normal(rng: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> Bf16Array:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return Bf16Array.from_f32(a)


@dataclass
class AttnInputs:
    cu_seqlens: np.ndarray
    grid: np.ndarray
    q: Bf16Array
    k: Bf16Array
    v: Bf16Array
    w_q: Bf16Array
    w_k: Bf16Array
    seed: int
    extra: Dict[str, object] = field(default_factory=dict)


def attention_inputs(cu_seqlens: np.ndarray, grid: np.ndarray, heads: int, head_dim: int,
                     seed: int) -> AttnInputs:
    """q, k, v ~ N(0,1) [N, H, D] then Q/K-norm gains 1 + N(0, 0.1) [D].
    Draw order: q, k, v, w_q, w_k."""
    n = int(cu_seqlens[-1])
    rng = np.random.default_rng(seed)
    q = _normal(rng, (n, heads, head_dim))
    k = _normal(rng, (n, heads, head_dim))
    v = _normal(rng, (n, heads, head_dim))
    w_q = _normal(rng, (head_dim,), std=0.1, mean=1.0)
    w_k = _normal(rng, (head_dim,), std=0.1, mean=1.0)
    return AttnInputs(np.asarray(cu_seqlens, np.int32), np.asarray(grid, np.int32),
                      q, k, v, w_q, w_k, seed)


def workload_attention_inputs(name: str) -> AttnInputs:
    w = WORKLOADS[name]
    cu, grid = pack(w.requests)
    return attention_inputs(cu, grid, w.heads, w.head_dim, w.seed)


def frame_local_attention_inputs(cu_seqlens: np.ndarray, heads: int, head_dim: int, seed: int,
                                 block: int = 1008, bonus: float = 12.0) -> AttnInputs:
    """Structured variant that makes attention peaked within blocks of tokens.

    q_t and k_t get mu * u_b added, with u_b a random unit vector per block of
    `block` consecutive tokens (one video frame of 24 x 42 latents) and head,
    and mu^2 = bonus * sqrt(head_dim), so keys of the same block gain about
    `bonus` in the scaled logit. Draw order: the i.i.d. q, k, v, gains as in
    attention_inputs, then u [num_blocks, H, D]. The shift is added in float32
    before the bf16 rounding of q and k."""
    n = int(cu_seqlens[-1])
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(size=(n, heads, head_dim), dtype=np.float32)
    k = rng.standard_normal(size=(n, heads, head_dim), dtype=np.float32)
    v = _normal(rng, (n, heads, head_dim))
    w_q = _normal(rng, (head_dim,), std=0.1, mean=1.0)
    w_k = _normal(rng, (head_dim,), std=0.1, mean=1.0)
    nb = (n + block - 1) // block
    u = rng.standard_normal(size=(nb, heads, head_dim), dtype=np.float32)
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    mu = np.float32(np.sqrt(bonus * np.sqrt(head_dim)))
    blk = np.arange(n) // block
    q += mu * u[blk]
    k += mu * u[blk]
    grid = np.zeros((n, 3), np.int32)
    return AttnInputs(np.asarray(cu_seqlens, np.int32), grid, Bf16Array.from_f32(q),
                      Bf16Array.from_f32(k), v, w_q, w_k, seed,
                      extra={"block": block, "bonus": bonus})


@dataclass
class BlockInputs:
    cu_seqlens: np.ndarray
    grid: np.ndarray
    x: Bf16Array
    cond: Bf16Array
    w_mod: Bf16Array
    w_qkv: Bf16Array
    w_o: Bf16Array
    q_norm: Bf16Array
    k_norm: Bf16Array
    w_gate: Bf16Array
    w_up: Bf16Array
    w_down: Bf16Array
    heads: int
    head_dim: int
    hidden: int
    ffn: int
    seed: int

    @property
    def weight_names(self):
        return ["w_mod", "w_qkv", "w_o", "q_norm", "k_norm", "w_gate", "w_up", "w_down"]


def block_inputs(cu_seqlens: np.ndarray, grid: np.ndarray, heads: int, head_dim: int,
                 ffn: int, seed: int, weight_std: float = 0.02) -> BlockInputs:
    """Activations N(0,1), linear weights N(0, weight_std), Q/K-norm gains
    1 + N(0, 0.1). Weights use the [out, in] layout. Draw order: x [N, C],
    cond [B, C], w_mod [6C, C], w_qkv [3C, C], w_o [C, C], q_norm [D],
    k_norm [D], w_gate [I, C], w_up [I, C], w_down [C, I]."""
    n = int(cu_seqlens[-1])
    b = len(cu_seqlens) - 1
    c = heads * head_dim
    rng = np.random.default_rng(seed)
    x = _normal(rng, (n, c))
    cond = _normal(rng, (b, c))
    w_mod = _normal(rng, (6 * c, c), std=weight_std)
    w_qkv = _normal(rng, (3 * c, c), std=weight_std)
    w_o = _normal(rng, (c, c), std=weight_std)
    q_norm = _normal(rng, (head_dim,), std=0.1, mean=1.0)
    k_norm = _normal(rng, (head_dim,), std=0.1, mean=1.0)
    w_gate = _normal(rng, (ffn, c), std=weight_std)
    w_up = _normal(rng, (ffn, c), std=weight_std)
    w_down = _normal(rng, (c, ffn), std=weight_std)
    return BlockInputs(np.asarray(cu_seqlens, np.int32), np.asarray(grid, np.int32), x, cond,
                       w_mod, w_qkv, w_o, q_norm, k_norm, w_gate, w_up, w_down,
                       heads, head_dim, c, ffn, seed)


def workload_block_inputs(name: str) -> BlockInputs:
    w = WORKLOADS[name]
    cu, grid = pack(w.requests)
    return block_inputs(cu, grid, w.heads, w.head_dim, w.ffn, w.seed)


def sample_rows(n: int, count: int, seed: int, include_edges: bool = True) -> np.ndarray:
    """Sorted distinct token indices for sampled parity checks."""
    rng = np.random.default_rng(seed + 7919)
    count = min(count, n)
    rows = set(rng.choice(n, size=count, replace=False).tolist())
    if include_edges and n > 0:
        rows.update({0, n - 1})
    return np.array(sorted(rows), dtype=np.int64)
