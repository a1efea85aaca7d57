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
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense fp4 / fp6 MFMA
ATTN_SRC = os.path.join(ROOT, "audio_diffusion_transformer_packed_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_block_10s_58k_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attention_flops(lengths, heads, head_dim):
    return float(sum(4.0 * L * L * heads * head_dim for L in lengths))


def gemm_flops(n, c, ffn, b):
    # qkv (3C), out-proj (C), gate+up (2I), down (I), modulation GEMV
    return 2.0 * n * c * (3 * c + c + 2 * ffn) + 2.0 * n * ffn * c + 2.0 * b * c * 6 * c


def block_roofline(n, c, ffn, heads, head_dim, lengths, b):
    """Roofline time of one block, sum over its kernels of max(FLOP / bf16
    peak, HBM bytes / HBM peak), in ms, with the per-kernel terms."""
    hd = heads * head_dim
    p, bw = PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9
    terms = {
        "modulation": (2.0 * b * c * 6 * c, 6 * c * c * 2.0),
        "adaln_x2": (0.0, 2 * 2.0 * n * c * 2),
        "qkv_gemm": (2.0 * n * c * 3 * c, 2.0 * (n * c + 3 * c * c + 3 * n * c)),
        "qk_rmsnorm_rope": (0.0, 4.0 * n * c * 2 + 12.0 * n),
        "attention": (attention_flops(lengths, heads, head_dim), 4.0 * n * hd * 2),
        "out_proj": (2.0 * n * c * c, 2.0 * (3 * n * c + c * c)),
        "swiglu_gemm": (2.0 * n * c * 2 * ffn, 2.0 * (n * c + 2 * ffn * c + n * ffn)),
        "down_gemm": (2.0 * n * ffn * c, 2.0 * (n * ffn + ffn * c + 2 * n * c)),
    }
    ms = {k: max(f / p, by / bw) * 1e3 for k, (f, by) in terms.items()}
    return sum(ms.values()), ms


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


def alternate(timer, fa, fb, n, rounds=4):
    """Average durations of two callables timed in alternating rounds of n
    launches each, so that drift of the shader clock during the run falls on
    both alike (used where their ratio is reported)."""
    ta = tb = 0.0
    for _ in range(rounds):
        ta += timer(fa, n)
        tb += timer(fb, n)
    return ta / rounds, tb / rounds


class Sampler:
    """Per-launch durations of a callable: a HIP event pair around each launch on
    the current torch stream. With flush=True a 512 MiB scratch buffer is written
    before every launch (outside the events), so an HBM-bound kernel reads its
    inputs from HBM rather than from the 256 MiB Infinity Cache."""

    def __init__(self, torch, flush_bytes=512 << 20, spin_cycles=2_000_000):
        self.torch = torch
        self.scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
        # a GPU-side busy wait (~1 ms) between the flush and the start event,
        # so the host has enqueued the event and the timed launch before the
        # GPU reaches them: the event pair then brackets the kernel alone,
        # not the host's launch overhead
        self.spin = getattr(torch.cuda, "_sleep", None)
        self.spin_cycles = spin_cycles

    def __call__(self, fn, n, flush):
        t = self.torch
        pairs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
                 for _ in range(n)]
        fn()
        t.cuda.synchronize()
        for i, (start, end) in enumerate(pairs):
            if flush:
                self.scratch.fill_(i & 0xff)
            if self.spin is not None:
                self.spin(self.spin_cycles)
            start.record()
            fn()
            end.record()
        t.cuda.synchronize()
        ms = np.array([start.elapsed_time(end) for start, end in pairs])
        return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
                "p90": float(np.percentile(ms, 90)), "n": n, "flush": flush}

    def stream(self, fns, single_ms, trials=5, target_ms=2.0, max_launches=48):
        """Mean duration per launch of back-to-back launches cycling over
        `fns` (each on its own copy of the inputs, enough copies that a
        copy's previous use lies more than 512 MiB of traffic back, so its
        inputs come from HBM, not the 256 MiB Infinity Cache), one event
        pair around each trial's launches. A long GPU-side busy wait before
        the start event lets the host enqueue the whole trial first, so the
        launches run back to back and the dispatch gap of a single launch
        (a few microseconds, large against a 20 us kernel) is amortised, as
        in a profiler's kernel durations. Median and spread over trials."""
        t = self.torch
        k = len(fns)
        launches = int(min(max_launches, max(2 * k, -(-target_ms // max(single_ms, 1e-3)))))
        launches = -(-launches // k) * k
        for f in fns:
            f()
        t.cuda.synchronize()
        per = []
        for _ in range(trials):
            start, end = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            if self.spin is not None:
                self.spin(8 * self.spin_cycles)
            start.record()
            for i in range(launches):
                fns[i % k]()
            end.record()
            t.cuda.synchronize()
            per.append(start.elapsed_time(end) / launches)
        per = np.array(per)
        return {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
                "p90": float(np.percentile(per, 90)), "n": launches * trials,
                "flush": f"back-to-back over {k} input copies"}


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


def _attn_chunk_worker(task):
    """One (head, 128-row query chunk) of the oracle's varlen attention, on
    q/k/v float32 [N, H, D] held in shared memory; BLAS single-threaded."""
    from multiprocessing import shared_memory
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass
    import oracle
    names, shape, cu, head, rows = task
    shms = [shared_memory.SharedMemory(name=nm) for nm in names]
    try:
        q, k, v = (np.ndarray(shape, dtype=np.float32, buffer=sh.buf) for sh in shms)
        out = oracle.attn_varlen_ref(q[:, head:head + 1], k[:, head:head + 1], v[:, head:head + 1], cu,
                                     rows=rows)
        return float(np.abs(out).sum())
    finally:
        for sh in shms:
            sh.close()


def rel_vs_float64_attention(o, q, k, v, cu, heads=(1, 11), groups=16, seed=351) -> float:
    """Relative Frobenius distance of attention output `o` [N, H, D] from
    float64 softmax attention (torch on the device, each row over its own
    segment's keys, scale 1/sqrt(D)) on `groups` sampled 32-row groups of two
    heads."""
    import torch
    n, d = o.shape[0], o.shape[2]
    rng = np.random.default_rng(seed)
    starts = sorted(set((32 * rng.integers(0, n // 32, groups)).tolist()))
    rows = np.array(sorted({t for t0 in starts for t in range(t0, min(n, t0 + 32))}))
    seg = np.searchsorted(np.asarray(cu), rows, side="right") - 1
    num = den = 0.0
    for h in heads:
        for s_ in np.unique(seg):
            r = torch.from_numpy(rows[seg == s_]).to(o.device)
            a, b = int(cu[s_]), int(cu[s_ + 1])
            qs = q[r, h].double()
            ks, vs = k[a:b, h].double(), v[a:b, h].double()
            ref = torch.softmax((qs @ ks.T.contiguous()) / np.sqrt(d), dim=1) @ vs
            got = o[r, h].double()
            num += float(((got - ref) ** 2).sum())
            den += float((ref ** 2).sum())
    return (num / den) ** 0.5


def cpu_attention_pool(wl, chunks_per_head=16):
    """The oracle's varlen attention (attn_varlen_ref, float64) on the
    workload's attention shape, timed over a process pool of one worker per
    host core, one task per (head, 128-row query chunk): every head, and
    `chunks_per_head` query chunks spread over the segment."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    import h3synth
    cu, _ = h3synth.pack(wl.requests)
    n, heads, d = int(cu[-1]), wl.heads, wl.head_dim
    inp = h3synth.attention_inputs(cu, np.zeros((n, 3), np.int32), heads, d, wl.seed)
    shms, names = [], []
    for a in (inp.q.f32, inp.k.f32, inp.v.f32):
        sh = shared_memory.SharedMemory(create=True, size=a.nbytes)
        np.ndarray(a.shape, dtype=np.float32, buffer=sh.buf)[...] = a
        shms.append(sh)
        names.append(sh.name)
    del inp
    try:
        starts = np.linspace(0, (n - 128) // 128, chunks_per_head).astype(np.int64) * 128
        tasks = [(names, (n, heads, d), cu, h, np.arange(t0, min(n, t0 + 128)))
                 for h in range(heads) for t0 in starts]
        workers = len(os.sched_getaffinity(0))
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            pool.map_async(_attn_chunk_worker, tasks[:workers]).get(timeout=300)   # workers up
            t0 = time.perf_counter()
            pool.map_async(_attn_chunk_worker, tasks, chunksize=1).get(timeout=600)
            dt = time.perf_counter() - t0
    finally:
        for sh in shms:
            sh.close()
            sh.unlink()
    rows = sum(t[4].size for t in tasks)
    flops = 4.0 * n * d * rows                      # 4 L D per (query row, head), one segment
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": (f"float64 numpy oracle attention (attn_varlen_ref) at {n} tokens x {heads} heads x {d}: "
                       f"{chunks_per_head} query chunks of 128 rows per head against the whole segment, "
                       f"{len(tasks)} (head, chunk) tasks over a pool of {workers} single-threaded worker "
                       f"processes; {flops / 1e12:.3f} TFLOP in {dt:.1f} s")}


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
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the other workloads (5 s attention, 15 s block, frame-local fp8)")
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
        if "single_launch_ms" in t:
            e["single_launch_ms"] = round(t["single_launch_ms"], 4)
        if flops is not None:
            e["tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
            e["frac_bf16_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
        if nbytes is not None:
            e["gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            e["frac_hbm_peak"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        stages[name] = e

    def hbm_stream(fns):
        """HBM-bound stage: back-to-back launches over input copies (`fns`,
        one callable per copy), with the single-launch median (event pair
        around one launch after a 512 MiB flush) kept beside it."""
        single = sampler(fns[0], stage_iters, True)
        t = sampler.stream(fns, single["median"])
        t["single_launch_ms"] = single["median"]
        return t

    if not args.no_stages:
        log("timing stages")
        mod = taps["mod"]
        it = stage_iters
        w = weights
        mfma = lambda fn: sampler(fn, it, False)

        # six copies of the 113 MB weight: a copy's previous use lies 565 MB back
        wmods = [w["w_mod"]] + [w["w_mod"].clone() for _ in range(5)]
        rec("modulation_gemv", hbm_stream([lambda wm=wm: ops.modulation(cond, wm) for wm in wmods]),
            nbytes=6 * c * c * 2 + b * c * 2 + b * 6 * c * 4)
        del wmods
        # two copies of x (each launch moves 712 MB)
        xs = [x, x.clone()]
        rec("adaln_rmsnorm_modulate",
            hbm_stream([lambda xx=xx: ops.adaln_rmsnorm_modulate(xx, mod[:, 0:c], mod[:, c:2 * c], cu_d, cu,
                                                                 out=taps["h"]) for xx in xs]),
            nbytes=2 * n * c * 2)
        del xs
        rec("qkv_gemm", mfma(lambda: ops.linear(taps["h"], w["w_qkv"])),
            flops=2.0 * n * c * 3 * c)
        # in place, on two copies of the qkv buffer (each launch moves 1.4 GB)
        qkv2s = [qkv.clone(), qkv.clone()]
        qk2 = [(t2[:, :hd].view(n, wl.heads, wl.head_dim), t2[:, hd:2 * hd].view(n, wl.heads, wl.head_dim))
               for t2 in qkv2s]
        rec("qk_rmsnorm_rope",
            hbm_stream([lambda p2=p2: ops.qk_rmsnorm_rope(p2[0], p2[1], w["q_norm"], w["k_norm"], grid_d, split)
                        for p2 in qk2]),
            nbytes=4 * n * c * 2 + 12 * n)
        del qkv2s, qk2
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

        # The vendor library (torch.nn.functional.linear -> hipBLASLt) on the
        # same four products, without the fused epilogues (SwiGLU: the gate
        # and up products as one [N, 2I] GEMM; the residual GEMMs: the plain
        # product), and the same products followed by the epilogue in torch
        # (the residual GEMMs: addcmul of the segment's gate row, one segment
        # here, given to torch in bf16 so that its elementwise kernel runs in
        # one dtype; SwiGLU: silu(gate) * up), the unfused path the fused
        # kernels replace.
        import torch.nn.functional as F
        w_gu = torch.cat([w["w_gate"], w["w_up"]], dim=0)
        ffn = wl.ffn
        lib_cmp = {}
        epi_out = torch.empty(n, c, dtype=torch.bfloat16, device=dev)
        gate_o = mod[0, 2 * c:3 * c].to(torch.bfloat16)
        gate_d = mod[0, 5 * c:6 * c].to(torch.bfloat16)

        def swiglu_lib():
            gu = F.linear(taps["h2"], w_gu)
            return F.silu(gu[:, :ffn]) * gu[:, ffn:]

        for nm, a_in, w_in, ours, with_epi in (
                ("qkv_gemm", taps["h"], w["w_qkv"], "qkv_gemm", None),
                ("out_proj", taps["o"], w["w_o"], "out_proj_gated_residual",
                 lambda: torch.addcmul(x, F.linear(taps["o"], w["w_o"]), gate_o, out=epi_out)),
                ("swiglu_gate_up", taps["h2"], w_gu, "swiglu_gemm", swiglu_lib),
                ("down", taps["a"], w["w_down"], "down_gated_residual",
                 lambda: torch.addcmul(taps["x1"], F.linear(taps["a"], w["w_down"]), gate_d, out=epi_out))):
            fl = 2.0 * a_in.shape[0] * a_in.shape[1] * w_in.shape[0]
            t = sampler(lambda: F.linear(a_in, w_in), it, False)
            e = {"library_ms": round(t["median"], 4),
                 "library_tflops": round(fl / (t["median"] * 1e-3) / 1e12, 2),
                 "fused_ms": stages[ours]["ms"],
                 "fused_over_library": round(t["median"] / stages[ours]["ms"], 4)}
            if with_epi is not None:
                te = sampler(with_epi, it, False)
                e["library_with_torch_epilogue_ms"] = round(te["median"], 4)
                e["fused_over_library_with_epilogue"] = round(te["median"] / stages[ours]["ms"], 4)
            lib_cmp[nm] = e
        del w_gu, epi_out, gate_o, gate_d
        stages["gemm_library_comparison"] = lib_cmp

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
            hbm_stream([lambda: ops.frames_to_uint8_bthwc(frames, out=frames_u8)]),   # 3.8 GB per launch
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
        fp8_attn(True)
        ms_fp8, ms_fp8_skip = alternate(timer, lambda: fp8_attn(False), lambda: fp8_attn(True), it)
        skipped = int(counts.sum().item())
        pairs = wl.heads * sum(((L + 31) // 32) * ((L + 63) // 64) for L in wl.lengths)
        qbufs = ops.fp8_quantize(qv, kv, vv, cu_d, cu)
        qws = torch.empty(max(1 << 20, ops.lib().h3_fp8_quantize_workspace_size(b, n, wl.heads)),
                          dtype=torch.uint8, device=dev)
        tq = hbm_stream([lambda: ops.fp8_quantize(qv, kv, vv, cu_d, cu, out=qbufs, workspace=qws)])   # 2 GB per launch
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
               "skip_cost_when_nothing_skipped": round(ms_fp8_skip / ms_fp8 - 1.0, 4),
               "skip_fraction": round(skipped / pairs, 5),
               "skip_threshold": 8.0}
        # accuracy of the dense fp8 output (skip off) against float64
        # attention on sampled rows, next to the literal 5e-2 relative bar:
        # on the block's q/k/v, and on the i.i.d. q/k/v of the
        # attn_fp8_10s_58k workload (the inputs of the parity tests)
        fp8_attn(False)
        rel = rel_vs_float64_attention(o8, qv, kv, vv, cu)
        w8 = h3synth.WORKLOADS["attn_fp8_10s_58k"]
        inp8 = h3synth.workload_attention_inputs(w8.name)
        q8, k8, v8 = dev_bf16(inp8.q), dev_bf16(inp8.k), dev_bf16(inp8.v)
        cu8 = inp8.cu_seqlens
        o8i = torch.empty_like(q8)
        ws8 = torch.empty(ops.attn_workspace_bytes(cu8, int(cu8[-1]), w8.heads, w8.head_dim, "fp8"),
                          dtype=torch.uint8, device=dev)
        ops.attn_varlen(q8, k8, v8, torch.from_numpy(cu8).to(dev), cu8, out=o8i, precision="fp8",
                        workspace=ws8)
        rel_iid = rel_vs_float64_attention(o8i, q8, k8, v8, cu8)
        del inp8, q8, k8, v8, o8i, ws8
        fp8["rel_frob_vs_float64_sampled"] = {
            "block_qkv": round(rel, 5), "iid_attn_fp8_10s_58k": round(rel_iid, 5),
            "rows": "16 sampled 32-row groups of heads 1 and 11"}
        fp8["literal_bar_5e-2_met"] = {"block_qkv": bool(rel <= 5e-2), "iid_attn_fp8_10s_58k": bool(rel_iid <= 5e-2)}
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
                if "single_launch_ms" in t:
                    e["single_launch_ms"] = round(t["single_launch_ms"], 4)
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
            xs = [x, x.clone()]
            mxrec("adaln_mx", hbm_stream([lambda xx=xx: ops.adaln_rmsnorm_modulate_mx(
                xx, mod[:, 0:c], mod[:, c:2 * c], cu_d, cu, out=h_mx) for xx in xs]),
                nbytes=n * c * 2 + n * c + n * c // 32)
            del xs
            mxrec("qkv_gemm_mx", sampler(lambda: ops.linear_mx(h_mx, wmx["w_qkv"]), it, False),
                  flops=2.0 * n * c * 3 * c)
            os_ = [taps["o"], taps["o"].clone()]
            mxrec("o_quantize_mx", hbm_stream([lambda oo=oo: ops.mx_quantize(oo, out=o_mx) for oo in os_]),
                  nbytes=n * c * 2 + n * c + n * c // 32)
            del os_
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

    # The same block with MXFP4 (OCP MX v1.0, E2M1) linears: weights
    # quantised once before timing; a step quantises its activations.
    mx4r = None
    if not args.no_mx:
        log("timing mxfp4 block")
        blk4 = ops.DitBlockMX4(weights, wl.heads, wl.head_dim, wl.ffn, split)
        ws4 = torch.empty(blk4.workspace_bytes(b, n), dtype=torch.uint8, device=dev)
        out4 = torch.empty_like(x)
        step4 = lambda: blk4.forward(x, cond, cu_d, cu, grid_d, out=out4, workspace=ws4)
        for _ in range(args.warmup):
            step4()
        ms4 = timer(step4, args.steps)
        st4 = {}
        if not args.no_stages:
            mod = taps["mod"]
            w4 = blk4.mx
            h4 = ops.mx4_quantize(taps["h"])
            o4 = ops.mx4_quantize(taps["o"])
            h24 = ops.mx4_quantize(taps["h2"])
            a4 = ops.mx4_quantize(taps["a"])
            y4 = torch.empty((n, 3 * c), dtype=torch.bfloat16, device=dev)
            ya = torch.empty((n, wl.ffn), dtype=torch.bfloat16, device=dev)
            yx = torch.empty_like(x)

            def rec4(name, t, flops=None, nbytes=None):
                e = {"ms": round(t["median"], 4), "p10_ms": round(t["p10"], 4), "p90_ms": round(t["p90"], 4),
                     "launches": t["n"], "mall_flushed": t["flush"]}
                if "single_launch_ms" in t:
                    e["single_launch_ms"] = round(t["single_launch_ms"], 4)
                if flops is not None:
                    tf = flops / (t["median"] * 1e-3) / 1e12
                    e["tflops"] = round(tf, 2)
                    e["frac_fp4_peak"] = round(tf / PEAK_FP4_TFLOPS, 4)
                if nbytes is not None:
                    gbs = nbytes / (t["median"] * 1e-3) / 1e9
                    e["gbs"] = round(gbs, 1)
                    e["frac_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
                st4[name] = e
            it = stage_iters
            hs = [taps["h"], taps["h"].clone()]
            rec4("h_quantize_mx4", hbm_stream([lambda hh=hh: ops.mx4_quantize(hh, out=h4) for hh in hs]),
                 nbytes=n * c * 2 + n * c // 2 + n * c // 32)
            del hs
            rec4("qkv_gemm_mx4", sampler(lambda: ops.linear_mx4(h4, w4["w_qkv"], out=y4), it, False),
                 flops=2.0 * n * c * 3 * c)
            rec4("out_proj_gated_residual_mx4", sampler(lambda: ops.linear_gated_residual_mx4(
                o4, w4["w_o"], x, mod[:, 2 * c:3 * c], cu_d, cu, out=yx), it, False), flops=2.0 * n * c * c)
            rec4("swiglu_gemm_mx4", sampler(lambda: ops.linear_swiglu_mx4(h24, w4["w_gate"], w4["w_up"], out=ya),
                                            it, False), flops=2.0 * n * c * 2 * wl.ffn)
            rec4("down_gated_residual_mx4", sampler(lambda: ops.linear_gated_residual_mx4(
                a4, w4["w_down"], taps["x1"], mod[:, 5 * c:6 * c], cu_d, cu, out=yx), it, False),
                flops=2.0 * n * wl.ffn * c)
            del h4, o4, h24, a4, y4, ya, yx
        mx4r = {"workload": f"{wl.name} with MXFP4 (OCP MX v1.0, E2M1, 32-element K blocks) linears",
                "block_ms": round(ms4, 4),
                "block_tflops": round((f_attn + f_gemm) / (ms4 * 1e-3) / 1e12, 2),
                "speedup_vs_bf16_block": round(ms_step / ms4, 4),
                "stages": st4}
        del blk4, ws4, out4

    # Other workloads of the method, timed as one leg each.
    legs = {}
    if not args.no_legs:
        rl_ms, rl_terms = block_roofline(n, c, wl.ffn, wl.heads, wl.head_dim, wl.lengths, b)
        legs["block_10s_58k_roofline"] = {"roofline_ms": round(rl_ms, 3),
                                          "frac_roofline": round(rl_ms / ms_step, 4),
                                          "terms_ms": {k: round(v, 4) for k, v in rl_terms.items()}}
        # attention only, 5 s clip: 32,260 tokens, 24 x 128, i.i.d. N(0,1)
        log("leg attn_5s_32k")
        w1 = h3synth.WORKLOADS["attn_5s_32k"]
        a1 = h3synth.workload_attention_inputs(w1.name)
        cu1 = a1.cu_seqlens
        q1, k1, v1 = dev_bf16(a1.q), dev_bf16(a1.k), dev_bf16(a1.v)
        cu1_d = torch.from_numpy(cu1).to(dev)
        o1 = torch.empty_like(q1)
        ws1 = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        f1 = attention_flops(w1.lengths, w1.heads, w1.head_dim)
        att1 = lambda: ops.attn_varlen(q1, k1, v1, cu1_d, cu1, out=o1, workspace=ws1)
        for _ in range(args.warmup):
            att1()
        ms1 = timer(att1, max(3, args.steps))
        legs["attn_5s_32k"] = {"workload": f"attn_5s_32k: one request of {int(cu1[-1])} tokens, "
                                           f"{w1.heads} heads x {w1.head_dim}, bf16",
                               "attention_ms": round(ms1, 4),
                               "attention_tflops": round(f1 / (ms1 * 1e-3) / 1e12, 2),
                               "attention_frac_bf16_peak": round(f1 / (ms1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del q1, k1, v1, o1, a1

        # 15 s clip: the whole block at 93,740 tokens
        log("leg block_15s_94k")
        w3 = h3synth.WORKLOADS["block_15s_94k"]
        b3 = h3synth.workload_block_inputs(w3.name)
        wt3 = {nm: dev_bf16(getattr(b3, nm)) for nm in ops.WEIGHT_NAMES}
        blk3 = ops.DitBlock(wt3, w3.heads, w3.head_dim, w3.ffn, h3synth.rope_split_for(w3.head_dim))
        cu3 = b3.cu_seqlens
        n3 = w3.total_tokens
        x3, cond3 = dev_bf16(b3.x), dev_bf16(b3.cond)
        cu3_d, grid3_d = torch.from_numpy(cu3).to(dev), torch.from_numpy(b3.grid).to(dev)
        out3 = torch.empty_like(x3)
        ws3 = torch.empty(blk3.workspace_bytes(len(cu3) - 1, n3), dtype=torch.uint8, device=dev)
        step3 = lambda: blk3.forward(x3, cond3, cu3_d, cu3, grid3_d, out=out3, workspace=ws3)
        for _ in range(args.warmup):
            step3()
        ms3 = timer(step3, args.steps)
        f3 = attention_flops(w3.lengths, w3.heads, w3.head_dim) + gemm_flops(n3, w3.hidden, w3.ffn, len(cu3) - 1)
        rl3, _ = block_roofline(n3, w3.hidden, w3.ffn, w3.heads, w3.head_dim, w3.lengths, len(cu3) - 1)
        legs["block_15s_94k"] = {"workload": f"block_15s_94k: {n3} tokens, same block dims",
                                 "block_ms": round(ms3, 4), "block_tflop": round(f3 / 1e12, 4),
                                 "block_tflops": round(f3 / (ms3 * 1e-3) / 1e12, 2),
                                 "roofline_ms": round(rl3, 3), "frac_roofline": round(rl3 / ms3, 4)}
        del x3, cond3, out3, ws3, wt3, blk3, b3
        torch.cuda.empty_cache()

        # fp8 attention with skip-softmax on the labelled frame-local variant
        # of the 10 s shape (q, k += mu u_frame per 1008-token block, a +12
        # logit bonus inside a block), skip off and on
        log("leg fp8 frame-local")
        a4 = h3synth.frame_local_attention_inputs(cu, wl.heads, wl.head_dim, seed=inp.seed)
        q4, k4, v4 = dev_bf16(a4.q), dev_bf16(a4.k), dev_bf16(a4.v)
        o4 = torch.empty_like(q4)
        ws4 = torch.empty(ops.attn_workspace_bytes(cu, n, wl.heads, wl.head_dim, "fp8"),
                          dtype=torch.uint8, device=dev)
        items4 = ops.attn_num_items(cu, wl.heads)
        cnt4 = torch.zeros(items4, dtype=torch.int32, device=dev)
        fp8_4 = lambda sk: ops.attn_varlen(q4, k4, v4, cu_d, cu, out=o4, precision="fp8", skip_softmax=sk,
                                           skip_counts=cnt4, workspace=ws4)
        fp8_4(False)
        fp8_4(True)
        ms4_off, ms4_on = alternate(timer, lambda: fp8_4(False), lambda: fp8_4(True), max(3, args.steps))
        pairs4 = wl.heads * sum(((L + 31) // 32) * ((L + 63) // 64) for L in wl.lengths)
        frac4 = int(cnt4.sum().item()) / pairs4
        legs["fp8_attention_frame_local"] = {
            "workload": f"{wl.name} shape, labelled frame-local variant (+12 logit bonus within 1008-token "
                        "blocks), fp8 e4m3 attention, skip threshold 8",
            "skip_off_ms": round(ms4_off, 4), "skip_on_ms": round(ms4_on, 4),
            "skip_fraction": round(frac4, 4), "speedup_from_skip": round(ms4_off / ms4_on, 4),
            "dense_equiv_tflops_skip_on": round(f_attn / (ms4_on * 1e-3) / 1e12, 2)}
        del q4, k4, v4, o4, ws4, a4
        torch.cuda.empty_cache()

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
        "mxfp4_linears": mx4r,
        "legs": legs,
        "timed_wall_s": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cb = cpu_attention_pool(wl)
        cb["block_sample"] = cpu_baseline(inp, wl)
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
