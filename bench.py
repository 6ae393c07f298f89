"""Benchmark of the quantized-KV decode hot path on one MI355X.

One step = append one new token to a cache (token accounting, tail-ring
write, and a flush-quantize when the window overflows by a whole group)
followed by single-query GQA decode attention over that cache, on the
Llama-3-8B attention shape: batch 8, 32 query / 8 KV heads, head_dim 128,
4096 cached tokens, int4 codes with per-channel Key and per-token Value fp16
scales, bf16 residual window of 128.

Steps rotate over independent caches whose combined footprint (> 512 MB) is
more than twice the 256 MB Infinity Cache, so the decode reads come from HBM.
Inputs are resident in HBM before timing starts.

Printed: one JSON line.  ``value`` = effective KV bytes read by the decode
attention per step (packed codes + Key scales + Value scales + bf16 tail +
queries) / measured time per step (append + decode, launch gaps included;
one HIP event pair around all timed steps).  ``roofline`` prices the decode
call alone (its two kernels): the same bytes over its average duration,
measured with one HIP event pair on the launch stream around as many
back-to-back decode calls over the same caches.
``cpu_baseline`` times the CPU oracle's decode attention on a bounded sample
of (batch, KV head) units of the same workload.

Other workloads (``--workload``) print their own line; the default run is
the decode workload above.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def decode_bytes(cfg, nq: int, nt: int, q_heads: int) -> int:
    """Algorithmic bytes one decode call must read (codes, scales, tail, q)."""
    B, H, D = cfg.batch, cfg.kv_heads, cfg.head_dim
    W = D * cfg.code_bits // 8
    es = 2 if cfg.kv_dtype == 0 else 4
    nseg = nq // cfg.group if cfg.group else None
    per_unit = 2 * nq * W + nq * 2 + 2 * nt * D * es
    per_unit += (nseg if nseg is not None else 0) * D * 2
    return B * H * per_unit + B * q_heads * D * es


def build_caches(w, n_caches, capacity, log):
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import KVCache, make_config

    cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=capacity,
                      code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
    caches = []
    for i in range(n_caches):
        s = ks.Stream(w, seed=i)
        k, v = ks.kv_pair(s, w.prefill)
        c = KVCache(cfg, zero=False)
        c.append(k.cuda(), v.cuda())
        caches.append(c)
        del k, v
    torch.cuda.synchronize()
    log(f"built {n_caches} caches of {w.prefill} tokens")
    return cfg, caches


def run_decode(args, log):
    import torch

    import kvq_synth as ks

    w = ks.LLAMA3_DECODE
    steps, warmup = args.steps, args.warmup
    capacity = w.prefill + (steps + warmup) // args.caches + 256
    cfg, caches = build_caches(w, args.caches, capacity, log)
    pool = 32
    s = ks.Stream(w, seed=10_000)
    new_k, new_v, qs = [], [], []
    for _ in range(pool):
        k, v = ks.kv_pair(s, 1)
        new_k.append(k.cuda())
        new_v.append(v.cuda())
        qs.append(ks.decode_query(s).cuda())
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    ws = caches[0].workspace(w.q_heads, 1)
    stream = torch.cuda.current_stream()

    def step(i):
        c = caches[i % len(caches)]
        c.append(new_k[i % pool], new_v[i % pool])
        return c

    for i in range(warmup):
        c = step(i)
        c.decode_attn(qs[i % pool], out, ws)
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_bytes = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        c = step(warmup + i)
        total_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
        c.decode_attn(qs[(warmup + i) % pool], out, ws)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    bytes_step = total_bytes / steps
    value = bytes_step / (ms_step * 1e-3) / 1e9

    # The decode call alone: the same caches, back-to-back calls on the launch
    # stream, one HIP event pair around all of them.
    dec_bytes = 0
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(steps):
        c = caches[i % len(caches)]
        dec_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
        c.decode_attn(qs[i % pool], out, ws)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / steps
    achieved = dec_bytes / steps / (dec_ms * 1e-3) / 1e9
    log(f"wall {wall:.3f}s for {steps} steps; {ms_step*1e3:.2f} us per step; decode call {dec_ms*1e3:.2f} us")
    res = {
        "metric": "decode-attn effective KV GB/s (% of HBM peak) + us/step, Llama-3-8B shape int4",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 3),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 MFMA (i32 acc) + f32 softmax", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "context": w.prefill,
                   "codes": f"int{w.code_bits}", "residual": w.residual, "group": w.group,
                   "caches_rotated": args.caches, "parallelism": "single-gpu"},
        "decode_call_us": round(dec_ms * 1e3, 3),
        "decode_bytes_per_step": int(bytes_step),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "kvq_decode_attn = decode_i8_kernel<128,4,4> + merge_kernel<128,4>"},
    }
    return res, (cfg, w)


def block_flops(nq_total: int, tq: int, q_heads: int, head_dim: int, batch: int = 1) -> float:
    """Algorithmic FLOPs of one causal block: QK^T and PV over N cached tokens
    plus the block's own visible tokens (query i sees i + 1 of them)."""
    pairs = tq * nq_total + tq * (tq + 1) // 2
    return 4.0 * batch * q_heads * head_dim * pairs


def run_video_block(args, log):
    """One causal block of 1024 queries against the 432000-token int2 cache."""
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import KVCache, make_config

    w = ks.VIDEO_BLOCK
    cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim,
                      capacity=w.prefill + 128, code_bits=w.code_bits, qmax=w.qmax,
                      residual=w.residual, group=w.group)
    s = ks.Stream(w, seed=0)
    k, v = ks.kv_pair(s, w.prefill)
    c = KVCache(cfg, zero=False)
    c.append(k.cuda(), v.cuda())
    del k, v
    q, kb, vb = (t.cuda() for t in ks.block_inputs(s, w.block_q))
    out = torch.empty(w.batch, w.block_q, w.q_heads, w.head_dim, device="cuda")
    ws = c.workspace(w.q_heads, w.block_q)
    stream = torch.cuda.current_stream()
    steps, warmup = max(1, args.steps // 20), max(1, args.warmup // 10)
    for _ in range(warmup):
        c.block_attn(q, kb, vb, out, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        c.block_attn(q, kb, vb, out, ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = block_flops(c.state.total, w.block_q, w.q_heads, w.head_dim, w.batch)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"video block: {ms:.3f} ms per block, {tflops:.1f} TFLOP/s")
    return {
        "metric": "causal block attention over the quantized cache, ms per block",
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/f16 MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "cached": c.state.total,
                   "block_q": w.block_q, "codes": f"int{w.code_bits}", "parallelism": "single-gpu"},
        "flops_per_block": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "kernel": "kvq_block_attn = block_kernel<128,2> + block_merge_kernel<128>"},
    }


def cpu_baseline_decode(budget_s: float, log):
    """Time the CPU oracle's decode attention on a bounded sample of units."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import kvq_synth as ks
    from oracle import attention as oatt
    from oracle.cache import KVQuantizationStrategies
    from quantized_kv_cache_kvq_amd import make_config

    w = ks.LLAMA3_DECODE
    s = ks.Stream(w, seed=0)
    k, v = ks.kv_pair(s, w.prefill)
    o = KVQuantizationStrategies(qmax=w.qmax, scale_storage="fp16", group=w.group)
    st = o.append_and_partition(None, k.float().numpy(), v.float().numpy(), w.residual)
    q = ks.decode_query(s).float().numpy()
    sigma = 1.0 / math.sqrt(w.head_dim)
    cfg = make_config(batch=1, kv_heads=1, head_dim=w.head_dim, capacity=w.prefill,
                      code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
    nq, nt = st["quantized_tokens"], st["key_residual"].shape[-2]
    unit_bytes = decode_bytes(cfg, nq, nt, w.q_heads // w.kv_heads)
    units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    # Whole decode calls (all 64 units) repeated until the budget is spent.
    with threadpool_limits(limits=1):
        calls = 0
        t = time.perf_counter()
        while True:
            oatt.decode_attention(st, q, sigma)
            calls += 1
            dt = time.perf_counter() - t
            if dt >= budget_s:
                break
    n = calls * len(units)
    log(f"cpu oracle: {calls} decode calls in {dt:.2f}s")
    return {"value": round(n * unit_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{calls} full fp64 decode-attention calls (restore + softmax over all "
                      f"{len(units)} (batch, KV head) units) of the Llama-3-8B int4 workload "
                      f"at {w.prefill} tokens, one thread, {dt:.1f} s; "
                      f"{dt / calls * 1e3:.1f} ms per call",
            "cpu": platform.processor() or platform.machine()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--caches", type=int, default=16)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--workload", choices=["llama3_decode", "video_block"], default="llama3_decode",
                    help="llama3_decode (default): the append + decode step; video_block: one "
                         "1024-query causal block against the 432000-token int2 cache")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import quantized_kv_cache_kvq_amd as kvq
    if not os.path.exists(kvq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    kvq.load()
    if args.workload == "video_block":
        res = run_video_block(args, log)
    else:
        res, _ = run_decode(args, log)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_decode(args.cpu_budget, log)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
