"""Benchmark of the packed joint audio-video DiT hot path on one MI355X.

One step = one full DiT block forward (h3_dit_block_forward: modulation,
AdaLN, QKV GEMM, Q/K RMSNorm + 3D RoPE, varlen attention, out-projection with
gated residual, AdaLN, SwiGLU GEMM, down GEMM with gated residual) over the
57,960-token packed sequence of a 10 s clip, inputs resident in HBM.

Prints ONE JSON line:
  value       whole-block throughput, algorithmic TFLOP/s (GEMMs + attention
              over valid tokens only, no padding) = block FLOPs / ms_per_step
  roofline    the dominant kernel (varlen attention) against bf16 dense MFMA
              peak, its average launch duration timed with HIP events on the
              stream it runs on
  stages      per-kernel timings: median and p10/p90 of >= 20 launches, each
              bracketed by HIP events; HBM-bound kernels run after a 512 MiB
              scratch write so they do not read from the 256 MiB MALL
  cpu_baseline the float64 oracle on the host cores, on a bounded sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-stages]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "varlen attention TFLOP/s + DiT-block ms at 58k packed tokens; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
ATTN_SRC = os.path.join(ROOT, "audio_diffusion_transformer_packed_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_block_10s_58k_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attention_flops(lengths, heads, head_dim):
    return float(sum(4.0 * L * L * heads * head_dim for L in lengths))


def gemm_flops(n, c, ffn, b):
    # qkv (3C), out-proj (C), gate+up (2I), down (I), modulation GEMV
    return 2.0 * n * c * (3 * c + c + 2 * ffn) + 2.0 * n * ffn * c + 2.0 * b * c * 6 * c


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != source_hash(ATTN_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


class Timer:
    """Average duration of a callable over n launches, with HIP events on the
    current torch stream (the stream the library enqueues on)."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, n):
        t = self.torch
        start, end = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        start.record()
        for _ in range(n):
            fn()
        end.record()
        t.cuda.synchronize()
        return start.elapsed_time(end) / n


class Sampler:
    """Per-launch durations of a callable: a HIP event pair around each launch on
    the current torch stream. With flush=True a 512 MiB scratch buffer is written
    before every launch (outside the events), so an HBM-bound kernel reads its
    inputs from HBM rather than from the 256 MiB Infinity Cache."""

    def __init__(self, torch, flush_bytes=512 << 20):
        self.torch = torch
        self.scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")

    def __call__(self, fn, n, flush):
        t = self.torch
        pairs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
                 for _ in range(n)]
        fn()
        t.cuda.synchronize()
        for i, (start, end) in enumerate(pairs):
            if flush:
                self.scratch.fill_(i & 0xff)
            start.record()
            fn()
            end.record()
        t.cuda.synchronize()
        ms = np.array([start.elapsed_time(end) for start, end in pairs])
        return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
                "p90": float(np.percentile(ms, 90)), "n": n, "flush": flush}


def cpu_baseline(inp, wl, rows_count=16):
    """The float64 oracle on a bounded sample of the same block: keys and values
    of all tokens plus the full block for `rows_count` sampled query rows."""
    import oracle
    from oracle import dit_block_rows_ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = os.cpu_count() or 1
    import h3synth
    n, c, ffn, heads, d = wl.total_tokens, wl.hidden, wl.ffn, wl.heads, wl.head_dim
    rows = h3synth.sample_rows(n, rows_count, inp.seed, include_edges=False)
    weights = {nm: getattr(inp, nm).f32 for nm in inp.weight_names}
    t0 = time.perf_counter()
    dit_block_rows_ref(inp.x.f32, inp.cond.f32, weights, inp.cu_seqlens, inp.grid, heads, d,
                       h3synth.rope_split_for(d), rows)
    dt = time.perf_counter() - t0
    r = rows.size
    L = n   # one segment
    flops = (2.0 * n * c * 2 * c                         # k, v projections, all tokens
             + r * (2.0 * c * c + 4.0 * L * c + 2.0 * c * c + 2.0 * c * 2 * ffn + 2.0 * ffn * c)
             + 2.0 * len(wl.requests) * c * 6 * c)
    del oracle
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": (f"float64 numpy oracle (dit_block_rows_ref): keys/values of all {n} tokens "
                       f"+ the whole block for {r} sampled query rows; {flops / 1e12:.3f} "
                       f"TFLOP algorithmic in {dt:.1f} s")}


def bsa_kept_flops(lists, lengths, head_dim, sparsity) -> float:
    """4 D x (query rows x kept keys), summed over heads and 256-row query
    blocks, from kept-block lists [H, T, stride] (row = first 64-token block
    of the query block)."""
    total = 0.0
    tile = 0
    for L in lengths:
        n_kb = (L + 63) // 64
        keep = max(1, n_kb - (n_kb * round(1000 * sparsity)) // 1000) if n_kb else 0
        for t0 in range(0, L, 256):
            rows = min(256, L - t0)
            blocks = lists[:, tile + t0 // 64, :keep]                      # [H, keep]
            keys = np.minimum(64, L - 64 * blocks).sum()
            total += 4.0 * head_dim * rows * float(keys)
        tile += n_kb
    return total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="block_10s_58k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-mx", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this hot path runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note, not built)"}))
        sys.exit(2)

    import torch
    import h3synth
    from audio_diffusion_transformer_packed_amd import ops

    dev = torch.device("cuda:0")
    wl = h3synth.WORKLOADS[args.workload]
    if wl.kind != "block":
        raise SystemExit("the bench step is a full block; pick a block workload")
    log(f"generating {wl.name}: {wl.total_tokens} tokens")
    inp = h3synth.workload_block_inputs(wl.name)
    split = h3synth.rope_split_for(wl.head_dim)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a.bits).view(np.int16)).to(dev).view(torch.bfloat16)

    weights = {nm: dev_bf16(getattr(inp, nm)) for nm in ops.WEIGHT_NAMES}
    blk = ops.DitBlock(weights, wl.heads, wl.head_dim, wl.ffn, split)
    cu = inp.cu_seqlens
    b, n, c = len(cu) - 1, wl.total_tokens, wl.hidden
    x = dev_bf16(inp.x)
    cond = dev_bf16(inp.cond)
    cu_d = torch.from_numpy(cu).to(dev)
    grid_d = torch.from_numpy(inp.grid).to(dev)
    out = torch.empty_like(x)
    ws = torch.empty(blk.workspace_bytes(b, n), dtype=torch.uint8, device=dev)
    step = lambda: blk.forward(x, cond, cu_d, cu, grid_d, out=out, workspace=ws)

    # Reference kernel for the HBM traffic counters: a plain 512 MiB device
    # copy reads and writes exactly 512 MiB; the FETCH_SIZE / WRITE_SIZE it
    # shows under rocprofv3 calibrates the counters of the attention kernel.
    copy_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(copy_src)
    copy_src.fill_(1)
    copy_dst.copy_(copy_src)
    del copy_src, copy_dst

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_wall = time.perf_counter()
    timer = Timer(torch)
    ms_step = timer(step, args.steps)
    t_wall = time.perf_counter() - t_wall

    f_attn = attention_flops(wl.lengths, wl.heads, wl.head_dim)
    f_gemm = gemm_flops(n, c, wl.ffn, b)
    block_tflops = (f_attn + f_gemm) / (ms_step * 1e-3) / 1e12

    # attention alone, on the block's own q/k/v (after norm + RoPE), same launch
    taps = blk.make_taps(b, n, dev)
    blk.forward(x, cond, cu_d, cu, grid_d, out=out, taps=taps, workspace=ws)
    qkv = taps["qkv"]
    hd = wl.heads * wl.head_dim
    qv = qkv[:, :hd].view(n, wl.heads, wl.head_dim)
    kv = qkv[:, hd:2 * hd].view(n, wl.heads, wl.head_dim)
    vv = qkv[:, 2 * hd:].view(n, wl.heads, wl.head_dim)
    o_att = taps["o"].view(n, wl.heads, wl.head_dim)
    attn_ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    attn = lambda: ops.attn_varlen(qv, kv, vv, cu_d, cu, out=o_att, workspace=attn_ws)
    attn()
    log("timing attention")
    ms_attn = timer(attn, max(3, args.steps))
    attn_tflops = f_attn / (ms_attn * 1e-3) / 1e12

    stages = {}
    sampler = Sampler(torch)
    stage_iters = max(20, args.steps)

    def rec(name, t, flops=None, nbytes=None):
        ms = t["median"]
        e = {"ms": round(ms, 4), "p10_ms": round(t["p10"], 4), "p90_ms": round(t["p90"], 4),
             "launches": t["n"], "mall_flushed": t["flush"]}
        if flops is not None:
            e["tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
            e["frac_bf16_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
        if nbytes is not None:
            e["gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            e["frac_hbm_peak"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        stages[name] = e

    if not args.no_stages:
        log("timing stages")
        mod = taps["mod"]
        it = stage_iters
        w = weights
        hbm = lambda fn: sampler(fn, it, True)
        mfma = lambda fn: sampler(fn, it, False)

        rec("modulation_gemv", hbm(lambda: ops.modulation(cond, w["w_mod"])),
            nbytes=6 * c * c * 2 + b * c * 2 + b * 6 * c * 4)
        rec("adaln_rmsnorm_modulate",
            hbm(lambda: ops.adaln_rmsnorm_modulate(x, mod[:, 0:c], mod[:, c:2 * c], cu_d, cu,
                                                   out=taps["h"])),
            nbytes=2 * n * c * 2)
        rec("qkv_gemm", mfma(lambda: ops.linear(taps["h"], w["w_qkv"])),
            flops=2.0 * n * c * 3 * c)
        qkv2 = qkv.clone()
        q2 = qkv2[:, :hd].view(n, wl.heads, wl.head_dim)
        k2 = qkv2[:, hd:2 * hd].view(n, wl.heads, wl.head_dim)
        rec("qk_rmsnorm_rope",
            hbm(lambda: ops.qk_rmsnorm_rope(q2, k2, w["q_norm"], w["k_norm"], grid_d, split)),
            nbytes=4 * n * c * 2 + 12 * n)
        del qkv2
        rec("attention_bf16", mfma(attn), flops=f_attn)
        rec("out_proj_gated_residual",
            mfma(lambda: ops.linear_gated_residual(taps["o"], w["w_o"], x, mod[:, 2 * c:3 * c],
                                                   cu_d, cu, out=taps["x1"])),
            flops=2.0 * n * c * c)
        rec("swiglu_gemm", mfma(lambda: ops.linear_swiglu(taps["h2"], w["w_gate"], w["w_up"])),
            flops=2.0 * n * c * 2 * wl.ffn)
        rec("down_gated_residual",
            mfma(lambda: ops.linear_gated_residual(taps["a"], w["w_down"], taps["x1"],
                                                   mod[:, 5 * c:6 * c], cu_d, cu,
                                                   out=taps["h2"])),
            flops=2.0 * n * wl.ffn * c)

    # Attention at one rank's share of an 8-way head split (3 of the 24 heads,
    # all 57,960 tokens): 681 work items on 256 CUs, where the last partial
    # wave of work items shows.
    if not args.no_stages:
        h_rank = max(1, wl.heads // 8)
        o_rank = torch.empty(n, h_rank, wl.head_dim, dtype=torch.bfloat16, device=dev)
        rank_attn = lambda: ops.attn_varlen(qv[:, :h_rank], kv[:, :h_rank], vv[:, :h_rank], cu_d,
                                            cu, out=o_rank, workspace=attn_ws)
        rec(f"attention_bf16_per_rank_h{h_rank}", sampler(rank_attn, stage_iters, False),
            flops=attention_flops(wl.lengths, h_rank, wl.head_dim))

    # Decoded-frame compaction (FP32 BCTHW -> uint8 BTHWC) at the 10 s clip's
    # 243 frames of 1344 x 768 RGB: 3.0 GB read, 0.75 GB written. Synthetic
    # frames uniform in [-1.1, 1.1] from a seeded torch generator.
    if not args.no_stages:
        gen = torch.Generator(device=dev)
        gen.manual_seed(inp.seed)
        frames = torch.rand((1, 3, 243, 768, 1344), generator=gen, device=dev) * 2.2 - 1.1
        frames_u8 = torch.empty((1, 243, 768, 1344, 3), dtype=torch.uint8, device=dev)
        rec("frames_to_uint8_bthwc",
            sampler(lambda: ops.frames_to_uint8_bthwc(frames, out=frames_u8), stage_iters, True),
            nbytes=frames.numel() * 5)
        del frames, frames_u8

    fp8 = None
    if not args.no_fp8:
        log("timing fp8 attention")
        it = max(3, args.steps)
        o8 = torch.empty_like(o_att)
        fp8_ws = torch.empty(ops.attn_workspace_bytes(cu, n, wl.heads, wl.head_dim, "fp8"),
                             dtype=torch.uint8, device=dev)
        n_items = ops.attn_num_items(cu, wl.heads)
        counts = torch.zeros(n_items, dtype=torch.int32, device=dev)

        def fp8_attn(skip):
            return ops.attn_varlen(qv, kv, vv, cu_d, cu, out=o8, precision="fp8",
                                   skip_softmax=skip, skip_counts=counts, workspace=fp8_ws)
        fp8_attn(False)
        ms_fp8 = timer(lambda: fp8_attn(False), it)
        fp8_attn(True)
        ms_fp8_skip = timer(lambda: fp8_attn(True), it)
        skipped = int(counts.sum().item())
        pairs = wl.heads * sum(((L + 31) // 32) * ((L + 63) // 64) for L in wl.lengths)
        qbufs = ops.fp8_quantize(qv, kv, vv, cu_d, cu)
        qws = torch.empty(max(1 << 20, ops.lib().h3_fp8_quantize_workspace_size(b, n, wl.heads)),
                          dtype=torch.uint8, device=dev)
        tq = sampler(lambda: ops.fp8_quantize(qv, kv, vv, cu_d, cu, out=qbufs, workspace=qws),
                     stage_iters, True)
        ms_q = tq["median"]
        q_bytes = 3 * n * c * 2 + n * c * 2 + 3 * n * c
        ms_k = ms_fp8 - ms_q
        fp8 = {"workload": "attn_fp8_10s_58k shape on the block's q/k/v",
               "quantize_ms": round(ms_q, 4),
               "quantize_gbs": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
               "quantize_frac_hbm_peak": round(q_bytes / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "attention_ms": round(ms_fp8, 4),
               "attention_dense_equiv_tflops": round(f_attn / (ms_fp8 * 1e-3) / 1e12, 2),
               "attention_kernel_ms": round(ms_k, 4),
               "attention_kernel_frac_fp8_peak": round(f_attn / (ms_k * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
               "skip_attention_ms": round(ms_fp8_skip, 4),
               "skip_fraction": round(skipped / pairs, 5),
               "skip_threshold": 8.0}
        rec("fp8_quantize", tq, nbytes=q_bytes)

    # Block-sparse attention (INT8 Q/K, FP8 V) at sparsity 0.8 on the same
    # q/k/v: the whole pass (quantise, select, attend). Algorithmic flops
    # count the kept keys only, from the kept-block lists of this input.
    bsa = None
    if not args.no_fp8:
        log("timing block-sparse attention")
        sp = 0.8
        bsa_ws = torch.empty(ops.lib().h3_attn_block_sparse_workspace_size(b, n, wl.heads, wl.head_dim, sp),
                             dtype=torch.uint8, device=dev)
        t_tiles = ops.fp8_num_tiles(cu)
        lists = torch.full((wl.heads, t_tiles, ops.attn_block_sparse_list_stride(cu, sp)), -1,
                           dtype=torch.int32, device=dev)
        o_bsa = torch.empty_like(o_att)
        bsa_fn = lambda: ops.attn_block_sparse(qv, kv, vv, cu_d, cu, sparsity=sp, out=o_bsa,
                                               kv_block_lists=lists, workspace=bsa_ws)
        bsa_fn()
        ms_bsa = timer(bsa_fn, max(3, args.steps))
        kept_flops = bsa_kept_flops(lists.cpu().numpy(), wl.lengths, wl.head_dim, sp)
        bsa = {"workload": f"{wl.name} q/k/v, block-sparse at sparsity {sp} (256-row query blocks, "
                           "64-key blocks, INT8 Q/K, FP8 V)",
               "attention_ms": round(ms_bsa, 4),
               "speedup_vs_fp8_dense": round(ms_fp8 / ms_bsa, 3),
               "speedup_vs_bf16_dense": round(ms_attn / ms_bsa, 3),
               "kept_key_fraction": round(kept_flops / f_attn, 4),
               "kept_tflops": round(kept_flops / (ms_bsa * 1e-3) / 1e12, 2),
               "kept_frac_int8_fp8_peak": round(kept_flops / (ms_bsa * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
        del bsa_ws, lists, o_bsa

    # The same block with MXFP8 (OCP MX, E4M3) linears: weights quantised once
    # before timing; a step quantises its activations inside the step.
    mxr = None
    if not args.no_mx:
        log("timing mxfp8 block")
        blk_mx = ops.DitBlockMX(weights, wl.heads, wl.head_dim, wl.ffn, split)
        ws_mx = torch.empty(blk_mx.workspace_bytes(b, n), dtype=torch.uint8, device=dev)
        out_mx = torch.empty_like(x)
        step_mx = lambda: blk_mx.forward(x, cond, cu_d, cu, grid_d, out=out_mx, workspace=ws_mx)
        for _ in range(args.warmup):
            step_mx()
        ms_mx = timer(step_mx, args.steps)
        mods = {}
        if not args.no_stages:
            mod = taps["mod"]
            wmx = blk_mx.mx
            h_mx = ops.adaln_rmsnorm_modulate_mx(x, mod[:, 0:c], mod[:, c:2 * c], cu_d, cu)
            o_mx = ops.mx_quantize(taps["o"])
            h2_mx = ops.adaln_rmsnorm_modulate_mx(taps["x1"], mod[:, 3 * c:4 * c], mod[:, 4 * c:5 * c],
                                                  cu_d, cu)
            a_mx = ops.linear_swiglu_mx(h2_mx, wmx["w_gate"], wmx["w_up"])
            x1_mx = torch.empty_like(x)
            x2_mx = torch.empty_like(x)

            def mxrec(name, t, flops=None, nbytes=None):
                e = {"ms": round(t["median"], 4), "p10_ms": round(t["p10"], 4), "p90_ms": round(t["p90"], 4),
                     "launches": t["n"], "mall_flushed": t["flush"]}
                if flops is not None:
                    tf = flops / (t["median"] * 1e-3) / 1e12
                    e["tflops"] = round(tf, 2)
                    e["frac_fp8_peak"] = round(tf / PEAK_FP8_TFLOPS, 4)
                if nbytes is not None:
                    gbs = nbytes / (t["median"] * 1e-3) / 1e9
                    e["gbs"] = round(gbs, 1)
                    e["frac_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
                mods[name] = e
            it = stage_iters
            mxrec("adaln_mx", sampler(lambda: ops.adaln_rmsnorm_modulate_mx(
                x, mod[:, 0:c], mod[:, c:2 * c], cu_d, cu, out=h_mx), it, True),
                nbytes=n * c * 2 + n * c + n * c // 32)
            mxrec("qkv_gemm_mx", sampler(lambda: ops.linear_mx(h_mx, wmx["w_qkv"]), it, False),
                  flops=2.0 * n * c * 3 * c)
            mxrec("o_quantize_mx", sampler(lambda: ops.mx_quantize(taps["o"], out=o_mx), it, True),
                  nbytes=n * c * 2 + n * c + n * c // 32)
            mxrec("out_proj_gated_residual_mx", sampler(lambda: ops.linear_gated_residual_mx(
                o_mx, wmx["w_o"], x, mod[:, 2 * c:3 * c], cu_d, cu, out=x1_mx), it, False),
                flops=2.0 * n * c * c)
            mxrec("swiglu_gemm_mx", sampler(lambda: ops.linear_swiglu_mx(h2_mx, wmx["w_gate"], wmx["w_up"],
                                                                         out=a_mx), it, False),
                  flops=2.0 * n * c * 2 * wl.ffn)
            mxrec("down_gated_residual_mx", sampler(lambda: ops.linear_gated_residual_mx(
                a_mx, wmx["w_down"], taps["x1"], mod[:, 5 * c:6 * c], cu_d, cu, out=x2_mx), it, False),
                flops=2.0 * n * wl.ffn * c)
            del h_mx, o_mx, h2_mx, a_mx, x1_mx, x2_mx
        mxr = {"workload": f"{wl.name} with MXFP8 (OCP MX v1.0, E4M3, 32-element K blocks) linears",
               "block_ms": round(ms_mx, 4),
               "block_tflops": round((f_attn + f_gemm) / (ms_mx * 1e-3) / 1e12, 2),
               "speedup_vs_bf16_block": round(ms_step / ms_mx, 4),
               "stages": mods}
        # The pages' lossy configuration: the same MXFP8 block with its
        # attention block-sparse (INT8 Q/K, FP8 V) at sparsity 0.8.
        blk_l = ops.DitBlockMX(weights, wl.heads, wl.head_dim, wl.ffn, split, attn_sparsity=0.8)
        ws_l = torch.empty(blk_l.workspace_bytes(b, n), dtype=torch.uint8, device=dev)
        step_l = lambda: blk_l.forward(x, cond, cu_d, cu, grid_d, out=out_mx, workspace=ws_l)
        for _ in range(args.warmup):
            step_l()
        ms_l = timer(step_l, args.steps)
        mxr["lossy_block_mxfp8_bsa"] = {
            "workload": f"{wl.name}, MXFP8 linears + block-sparse attention at sparsity 0.8",
            "block_ms": round(ms_l, 4), "speedup_vs_bf16_block": round(ms_step / ms_l, 3),
            "speedup_vs_mxfp8_block": round(ms_mx / ms_l, 3)}
        del blk_mx, ws_mx, out_mx, blk_l, ws_l

    traffic = load_traffic()
    result = {
        "metric": METRIC,
        "value": round(block_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": n, "segments": b, "hidden": c,
                   "heads": wl.heads, "head_dim": wl.head_dim, "ffn": wl.ffn,
                   "seed": inp.seed},
        "block_ms": round(ms_step, 4),
        "block_tflop": round((f_attn + f_gemm) / 1e12, 4),
        "attention_tflops": round(attn_tflops, 2),
        "attention_ms": round(ms_attn, 4),
        "attention_frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "block_frac_bf16_peak": round(block_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": "attn_bf16_kernel<128>", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "stages": stages,
        "fp8_attention": fp8,
        "block_sparse_attention": bsa,
        "mxfp8_linears": mxr,
        "timed_wall_s": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(inp, wl)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
