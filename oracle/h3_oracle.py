"""Float64 CPU oracle for the packed joint audio-video DiT hot path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline leg may import or call this module; the product path never does. It
shares no code with the HIP library and imports nothing from it.

Everything here is the plain definition of what the hot path computes,
written in numpy float64 on the exact (bf16-valued) inputs, with no rounding
of intermediates and no blocking beyond chunking rows to bound memory.

Sources, cited by page title and section:
  [FastH3-EN] "MiniMax H3 FastH3 real-time serving with vLLM-Omni"
      - "System-wide optimizations in vLLM-Omni", bullet "Long-sequence
        attention & communication": text, audio and video tokens of one
        request are packed into one long sequence and only valid tokens are
        processed (no padding).
      - same section, bullet "Fused DiT operators": RMSNorm, RoPE,
        modulation, normalization and SwiGLU are the per-block operators.
  [FastH3-ZH] "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长"
      - section "融合 DiT 算子" (fused DiT operators): RMSNorm, RoPE, SwiGLU
        and the residual connection; Q/K normalisation merged with RoPE;
        SwiGLU in place of separate SiLU and multiply.
      - section "长序列注意力与通信优化" (long-sequence attention): a packed
        sequence of about 58k tokens, attention over valid tokens only.

The pages give operator names, not equations. Where they are silent this
module takes the plainest reading (all of them listed with the design notes):
  * block: single-stream pre-norm AdaLN-Zero DiT block, one weight set shared
    by all modalities, modulation from one linear map of a per-request
    conditioning vector, chunks (shift1, scale1, gate1, shift2, scale2, gate2);
  * RMSNorm(z) = z / sqrt(mean(z^2) + eps), no gain on the AdaLN norms,
    per-head gain [D] on the Q/K norms; modulate as norm*(1+scale)+shift;
  * 3D RoPE over (t, h, w) with per-axis dims split, interleaved pairs
    (2j, 2j+1) inside each axis's slice, angle pos * theta^(-2j/d_axis);
  * attention is non-causal inside a segment, none across segments, scale
    1/sqrt(D).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence

import numpy as np

_F = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=_F)


def bf16_round(a) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even), in float64.

    Used only by the storage emulation of the block (see dit_block_ref); the
    exact oracle never rounds. Finite inputs within the bf16 range.
    """
    a = _f64(a)
    m, e = np.frexp(a)                  # a = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)   # np.round: ties to even


def _identity(a):
    return a


# --------------------------------------------------------------------------
# Packed-sequence bookkeeping  ([FastH3-EN] long-sequence attention bullet:
# padding is removed, so every index below refers to valid tokens only)
# --------------------------------------------------------------------------

def check_cu_seqlens(cu: Sequence[int]) -> np.ndarray:
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be 1-D with at least one entry")
    if cu[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    return cu


def segment_ids(cu: Sequence[int]) -> np.ndarray:
    """seg(t) = s for cu[s] <= t < cu[s+1]; int32[N]."""
    cu = check_cu_seqlens(cu)
    n = int(cu[-1])
    seg = np.empty(n, dtype=np.int32)
    for s in range(cu.size - 1):
        seg[cu[s]:cu[s + 1]] = s
    return seg


def tile_offsets(cu: Sequence[int], block_m: int) -> np.ndarray:
    """tile_cu[s+1] = tile_cu[s] + ceil(L_s / block_m); int32[B+1]."""
    cu = check_cu_seqlens(cu)
    out = np.zeros(cu.size, dtype=np.int64)
    for s in range(cu.size - 1):
        length = int(cu[s + 1] - cu[s])
        out[s + 1] = out[s] + (length + block_m - 1) // block_m
    return out.astype(np.int32)


def schedule_ref(cu: Sequence[int], num_heads: int, block_m: int) -> np.ndarray:
    """Attention work list: one item per (head, segment, query tile).

    Item = (head, segment, first query token (absolute index), rows in tile).
    Order: segments by descending length (ties by ascending index), then
    head ascending, then query tile ascending. Empty segments give no item.
    Returns int32[count, 4].
    """
    cu = check_cu_seqlens(cu)
    lengths = [int(cu[s + 1] - cu[s]) for s in range(cu.size - 1)]
    order = sorted(range(len(lengths)), key=lambda s: (-lengths[s], s))
    items = []
    for s in order:
        length = lengths[s]
        for h in range(num_heads):
            for off in range(0, length, block_m):
                items.append((h, s, int(cu[s]) + off, min(block_m, length - off)))
    return np.array(items, dtype=np.int32).reshape(-1, 4)


# --------------------------------------------------------------------------
# Norms and positional encoding  ([FastH3-ZH] fused DiT operators: RMSNorm,
# RoPE, Q/K normalisation merged with RoPE)
# --------------------------------------------------------------------------

def rmsnorm(z, eps: float) -> np.ndarray:
    """z / sqrt(mean(z^2) + eps) over the last axis."""
    z = _f64(z)
    return z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)


def rope_3d(x, pos, split: Sequence[int], theta: float) -> np.ndarray:
    """Rotate interleaved pairs of each axis slice by pos_axis * theta^(-2j/d).

    x: [..., D]; pos: integer positions [..., 3] broadcastable against x's
    leading axes. Axis a occupies dims [o_a, o_a + d_a) with o = (0, d_t,
    d_t + d_h); pair j of that slice is (o_a + 2j, o_a + 2j + 1) and maps
    (u, v) -> (u cos phi - v sin phi, u sin phi + v cos phi).
    """
    x = _f64(x)
    pos = np.asarray(pos)
    if sum(split) != x.shape[-1] or any(d % 2 for d in split):
        raise ValueError("RoPE split must be even and sum to the head dim")
    out = x.copy()
    off = 0
    for a, d in enumerate(split):
        j = np.arange(d // 2, dtype=_F)
        inv_freq = np.power(_F(theta), -2.0 * j / d)
        phi = _f64(pos[..., a])[..., None] * inv_freq
        c, s = np.cos(phi), np.sin(phi)
        u = x[..., off + 0:off + d:2]
        v = x[..., off + 1:off + d:2]
        out[..., off + 0:off + d:2] = u * c - v * s
        out[..., off + 1:off + d:2] = u * s + v * c
        off += d
    return out


def qk_norm_rope_ref(q, k, w_q, w_k, grid, split: Sequence[int], theta: float,
                     eps: float):
    """Per token and head: RoPE(RMSNorm_D(q) * w_q), same for k with w_k.

    q, k: [N, H, D]; w_q, w_k: [D] gains shared across heads;
    grid: int [N, 3] positions (t, h, w).
    """
    pos = np.asarray(grid)[:, None, :]
    qn = rmsnorm(q, eps) * _f64(w_q)
    kn = rmsnorm(k, eps) * _f64(w_k)
    return rope_3d(qn, pos, split, theta), rope_3d(kn, pos, split, theta)


# --------------------------------------------------------------------------
# Varlen joint attention  ([FastH3-EN] long-sequence attention bullet and
# [FastH3-ZH] long-sequence attention section: attention over the packed
# valid tokens, full inside a request, none across requests)
# --------------------------------------------------------------------------

def attn_varlen_ref(q, k, v, cu: Sequence[int], scale: Optional[float] = None,
                    rows: Optional[Sequence[int]] = None, chunk: int = 256) -> np.ndarray:
    """O = softmax(Q K^T * scale) V per (segment, head); non-causal.

    q, k, v: [N, H, D]. scale defaults to 1/sqrt(D). With `rows`, only those
    query tokens are computed (each still attends to its whole segment) and
    the result has shape [len(rows), H, D]; otherwise [N, H, D].
    Softmax is exp(S - rowmax) / sum.
    """
    cu = check_cu_seqlens(cu)
    q = np.asarray(q)
    n, heads, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seg = segment_ids(cu)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, heads, d), dtype=_F)
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seg[rows] == s)[0] if rows.size else np.zeros(0, np.int64)
        if b == a or sel.size == 0:
            continue
        ks = _f64(k[a:b])
        vs = _f64(v[a:b])
        for c0 in range(0, sel.size, chunk):
            idx = sel[c0:c0 + chunk]
            qs = _f64(q[rows[idx]])
            for h in range(heads):
                sc = (qs[:, h, :] @ ks[:, h, :].T) * scale
                p = np.exp(sc - sc.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                out[idx, h, :] = p @ vs[:, h, :]
    return out


# --------------------------------------------------------------------------
# AdaLN modulation, SwiGLU, gated residual  ([FastH3-EN] fused DiT operators
# bullet: modulation + normalization; [FastH3-ZH] fused DiT operators: SwiGLU
# instead of separate SiLU and multiply, residual connection)
# --------------------------------------------------------------------------

MOD_CHUNKS = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")


def modulation_ref(cond, w_mod) -> np.ndarray:
    """mod[b] = cond[b] . W_mod^T, [B, 6C] (no bias, no activation)."""
    return _f64(cond) @ _f64(w_mod).T


def split_modulation(mod, hidden: int) -> Dict[str, np.ndarray]:
    mod = _f64(mod)
    return {name: mod[:, i * hidden:(i + 1) * hidden] for i, name in enumerate(MOD_CHUNKS)}


def adaln_modulate_ref(x, shift, scale, seg, eps: float) -> np.ndarray:
    """h_t = RMSNorm(x_t) * (1 + scale[seg(t)]) + shift[seg(t)]."""
    seg = np.asarray(seg)
    return rmsnorm(x, eps) * (1.0 + _f64(scale)[seg]) + _f64(shift)[seg]


def silu(z) -> np.ndarray:
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_ref(h, w_gate, w_up) -> np.ndarray:
    """a = silu(h W_gate^T) * (h W_up^T)."""
    h = _f64(h)
    return silu(h @ _f64(w_gate).T) * (h @ _f64(w_up).T)


def gated_residual_ref(x, gate, y, seg) -> np.ndarray:
    """x + gate[seg(t)] * y."""
    return _f64(x) + _f64(gate)[np.asarray(seg)] * _f64(y)


# --------------------------------------------------------------------------
# The DiT block
# --------------------------------------------------------------------------

def _split_heads(qkv: np.ndarray, heads: int, head_dim: int):
    c = heads * head_dim
    n = qkv.shape[0]
    q = qkv[:, 0:c].reshape(n, heads, head_dim)
    k = qkv[:, c:2 * c].reshape(n, heads, head_dim)
    v = qkv[:, 2 * c:3 * c].reshape(n, heads, head_dim)
    return q, k, v


def dit_block_ref(x, cond, weights: Dict[str, np.ndarray], cu: Sequence[int], grid,
                  heads: int, head_dim: int, rope_split: Sequence[int],
                  rope_theta: float = 10000.0, eps: float = 1e-6,
                  emulate_bf16_storage: bool = False,
                  linear_quant: Optional[Callable] = None,
                  attention: Optional[Callable] = None) -> Dict[str, np.ndarray]:
    """One block over the whole packed sequence; returns every intermediate.

    With emulate_bf16_storage, every intermediate that the device path stores
    between kernels is rounded to bf16 (h, qkv, q/k after norm + RoPE, o, x1,
    h2, a, x2) and mod to float32; all arithmetic in between stays float64.
    This models the storage precision of the path, not its exact value.

    linear_quant (e.g. mx_linear.mx_fake_quant) replaces every operand of
    the four block linears by its quantised value: the weights, and the
    activations h, o, h2, a where they enter a linear. h, h2 and a are
    quantised from their unrounded values (the producing kernels quantise
    in registers), o from its stored value. The returned h, o, h2, a are the
    values the linears consumed.

    attention (default attn_varlen_ref) is called as attention(q, k, v, cu)
    on [N, H, D] arrays and returns o [N, H, D]; block_sparse_attention's
    emulation plugs in here for the pages' lossy configuration ("MiniMax H3
    on Ascend 950PR / 950DT", recommended lossy configuration: EQBSA with
    MXFP8).

    h   = RMSNorm(x)(1+scale1)+shift1
    qkv = h W_qkv^T                   (q | k | v, each head-major [H*D])
    q,k = RoPE(RMSNorm_D(.) * gain)
    o   = varlen attention(q, k, v)
    x1  = x + gate1 * (o W_o^T)
    h2  = RMSNorm(x1)(1+scale2)+shift2
    a   = silu(h2 W_gate^T) * (h2 W_up^T)
    x2  = x1 + gate2 * (a W_down^T)
    """
    st = bf16_round if emulate_bf16_storage else _identity
    lq = linear_quant
    act = (lambda z: lq(z)) if lq else st          # activation entering a linear
    wt = (lambda nm: lq(_f64(weights[nm]))) if lq else (lambda nm: _f64(weights[nm]))
    x = _f64(x)
    n, c = x.shape
    seg = segment_ids(cu)
    mod = modulation_ref(cond, weights["w_mod"])
    if emulate_bf16_storage:
        mod = mod.astype(np.float32).astype(_F)
    m = split_modulation(mod, c)
    h = act(adaln_modulate_ref(x, m["shift1"], m["scale1"], seg, eps))
    qkv = st(h @ wt("w_qkv").T)
    q, k, v = _split_heads(qkv, heads, head_dim)
    qr, kr = qk_norm_rope_ref(q, k, weights["q_norm"], weights["k_norm"], grid, rope_split,
                              rope_theta, eps)
    qr, kr = st(qr), st(kr)
    o = st((attention or attn_varlen_ref)(qr, kr, v, cu).reshape(n, c))
    if lq:
        o = lq(o)
    x1 = st(gated_residual_ref(x, m["gate1"], o @ wt("w_o").T, seg))
    h2 = act(adaln_modulate_ref(x1, m["shift2"], m["scale2"], seg, eps))
    a = act(swiglu_ref(h2, wt("w_gate"), wt("w_up")))
    x2 = st(gated_residual_ref(x1, m["gate2"], a @ wt("w_down").T, seg))
    return {"mod": mod, "h": h, "qkv": qkv, "q": qr.reshape(n, c), "k": kr.reshape(n, c),
            "v": v.reshape(n, c), "o": o, "x1": x1, "h2": h2, "a": a, "x2": x2}


def dit_block_rows_ref(x, cond, weights: Dict[str, np.ndarray], cu: Sequence[int], grid,
                       heads: int, head_dim: int, rope_split: Sequence[int], rows,
                       rope_theta: float = 10000.0, eps: float = 1e-6,
                       token_chunk: int = 4096,
                       emulate_bf16_storage: bool = False,
                       linear_quant: Optional[Callable] = None) -> Dict[str, np.ndarray]:
    """The same block for the sampled token indices `rows` only (exact, or
    with the storage emulation and linear quantisation of dit_block_ref;
    both quantisations act along K, per row, so sampling rows is exact).

    Keys and values of every token of the segments that hold a sampled row
    are computed (a sampled row attends to its whole segment); everything
    else is computed for the sampled rows alone. Outputs have len(rows)
    leading rows. Memory is bounded by processing tokens in chunks.
    """
    st = bf16_round if emulate_bf16_storage else _identity
    lq = linear_quant
    act = (lambda z: lq(z)) if lq else st
    wt = (lambda w: lq(w)) if lq else (lambda w: w)
    cu = check_cu_seqlens(cu)
    x32 = np.asarray(x)
    n, c = x32.shape
    rows = np.asarray(rows, dtype=np.int64)
    seg = segment_ids(cu)
    grid = np.asarray(grid)
    mod = modulation_ref(cond, weights["w_mod"])
    if emulate_bf16_storage:
        mod = mod.astype(np.float32).astype(_F)
    m = split_modulation(mod, c)
    w_qkv = wt(_f64(weights["w_qkv"]))
    w_q, w_k, w_v = w_qkv[0:c], w_qkv[c:2 * c], w_qkv[2 * c:3 * c]
    wq_t, wk_t, wv_t = w_q.T.copy(), w_k.T.copy(), w_v.T.copy()

    def project(tok):
        return act(adaln_modulate_ref(x32[tok], m["shift1"], m["scale1"], seg[tok], eps))

    out_o = np.zeros((rows.size, heads, head_dim), dtype=_F)
    for s in np.unique(seg[rows]) if rows.size else []:
        a, b = int(cu[s]), int(cu[s + 1])
        kk = np.empty((b - a, heads, head_dim), dtype=_F)
        vv = np.empty((b - a, heads, head_dim), dtype=_F)
        for t0 in range(a, b, token_chunk):
            tok = np.arange(t0, min(b, t0 + token_chunk))
            h = project(tok)
            k_raw = st(h @ wk_t).reshape(tok.size, heads, head_dim)
            vv[t0 - a:t0 - a + tok.size] = st(h @ wv_t).reshape(tok.size, heads, head_dim)
            kn = rmsnorm(k_raw, eps) * _f64(weights["k_norm"])
            kk[t0 - a:t0 - a + tok.size] = st(rope_3d(kn, grid[tok][:, None, :], rope_split,
                                                       rope_theta))
        sel = np.nonzero(seg[rows] == s)[0]
        tok = rows[sel]
        h = project(tok)
        q_raw = st(h @ wq_t).reshape(tok.size, heads, head_dim)
        qn = rmsnorm(q_raw, eps) * _f64(weights["q_norm"])
        qq = st(rope_3d(qn, grid[tok][:, None, :], rope_split, rope_theta))
        local_cu = [0, b - a]
        # attention of the sampled queries against the whole segment
        q_full = np.zeros((b - a, heads, head_dim), dtype=_F)
        q_full[tok - a] = qq
        out_o[sel] = attn_varlen_ref(q_full, kk, vv, local_cu, rows=tok - a)

    o = st(out_o.reshape(rows.size, c))
    if lq:
        o = lq(o)
    segr = seg[rows]
    xr = _f64(x32[rows])
    h = act(adaln_modulate_ref(xr, m["shift1"], m["scale1"], segr, eps))
    x1 = st(gated_residual_ref(xr, m["gate1"], o @ wt(_f64(weights["w_o"])).T, segr))
    h2 = act(adaln_modulate_ref(x1, m["shift2"], m["scale2"], segr, eps))
    a = act(swiglu_ref(h2, wt(_f64(weights["w_gate"])), wt(_f64(weights["w_up"]))))
    x2 = st(gated_residual_ref(x1, m["gate2"], a @ wt(_f64(weights["w_down"])).T, segr))
    return {"mod": mod, "h": h, "o": o, "x1": x1, "h2": h2, "a": a, "x2": x2}


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in float64."""
    got, ref = _f64(got), _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)
