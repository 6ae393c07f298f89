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
measured with one HIP event pair on the launch stream around back-to-back
replays of a HIP graph that holds one decode call per cache (the eager
back-to-back figure, which includes host launch cost, is reported beside it).
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

# HBM bytes per call from separate rocprofv3 --pmc passes of FETCH_SIZE and
# WRITE_SIZE over the same commands bench.py runs, each scaled by what the
# counter reads for the hbm_copy workload's known 256 MiB read + 256 MiB
# write (FETCH_SIZE x 2, WRITE_SIZE x 1).  Each describes the kernels named
# in profiles/ and is None while those kernels have changed since the
# counters were taken.
DECODE_CALL_TRAFFIC = 39_638_179     # decode_i8_kernel, 4096-token Llama-3-8B shape (algorithmic 37.78 MB)
LONG_CALL_TRAFFIC = 140_358_073      # one 131072-token layer (algorithmic 138.8 MB)
# 128 appends (16 flushes + 128 window copies) and one block-attention call
# (block_kernel + block_merge_kernel).
APPEND_RUN_TRAFFIC = {4: 444_055_424, 8: 479_014_967}
BLOCK_CALL_TRAFFIC = 2_067_551_539    # the cache is streamed once per query-row tile
PAGED_CALL_TRAFFIC = 43_744_240      # paged decode, ragged lengths (algorithmic 41.42 MB)
PAGED_BLOCK_CALL_TRAFFIC = 2_180_594_893  # the video block over a paged cache


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
    capacity = w.prefill + (3 * steps + warmup) // args.caches + 128 + 256
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

    # A step appends one token to a cache and attends with the new query over
    # the whole cache, the new token included: one kvq_decode_step call.
    def step(i):
        c = caches[i % len(caches)]
        c.decode_step(new_k[i % pool], new_v[i % pool], qs[i % pool], out, ws)
        return c

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_bytes = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        c = step(warmup + i)
        total_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    bytes_step = total_bytes / steps
    value = bytes_step / (ms_step * 1e-3) / 1e9

    # The same step as two calls (kvq_append, then kvq_decode_attn), for reference.
    t_bytes = 0
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        c = caches[i % len(caches)]
        c.append(new_k[i % pool], new_v[i % pool])
        t_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
        c.decode_attn(qs[i % pool], out, ws)
    end.record(stream)
    torch.cuda.synchronize()
    two_call_ms = start.elapsed_time(end) / steps

    # The decode call alone, eager: the same caches, back-to-back calls on the
    # launch stream, one HIP event pair around all of them (the host-side
    # launch cost of each call is included when it exceeds the GPU time).
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
    eager_ms = d0.elapsed_time(d1) / steps

    # The decode call as a serving loop issues it: one call per cache captured
    # into a HIP graph, replayed back to back (GPU time, no host launch cost).
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    g_bytes = 0
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i, c in enumerate(caches):
                g_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
                c.decode_attn(qs[i % pool], out, ws, stream=cap)
    stream.wait_stream(cap)
    replays = max(2, steps // len(caches))
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(replays):
        graph.replay()
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / (replays * len(caches))
    achieved = g_bytes / len(caches) / (dec_ms * 1e-3) / 1e9

    # Steps through a flush, as in a real decode loop with G = 128 (timed last,
    # so that the decode-call figures above see caches of about 4096 tokens):
    # 128 more steps per cache, round robin over the caches (each cache's window,
    # 128..255 tokens, reaches 256 exactly once and flushes 128 tokens).
    flush_rounds = 128
    f_bytes, f0 = 0, sum(c.state.segments for c in caches)
    torch.cuda.synchronize()
    start.record(stream)
    for r in range(flush_rounds):
        for j in range(len(caches)):
            c = step(r * len(caches) + j)
            f_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
    end.record(stream)
    torch.cuda.synchronize()
    flush_steps = flush_rounds * len(caches)
    flushes = sum(c.state.segments for c in caches) - f0
    flush_ms = start.elapsed_time(end) / flush_steps

    # The same steps captured in one HIP graph, as a serving loop that replays
    # a captured step sequence would run them: 8 steps per cache captured once
    # (the host-side accounting runs at capture).  Replays repeat the same
    # steps on the same slots, so only the first leaves the cache the calls
    # describe; the timing does not depend on the values.
    g_steps = 8 * len(caches)
    gs_bytes = 0
    step_graph = torch.cuda.CUDAGraph()
    cap2 = torch.cuda.Stream()
    cap2.wait_stream(stream)
    with torch.cuda.stream(cap2):
        with torch.cuda.graph(step_graph, stream=cap2):
            for i in range(g_steps):
                c = caches[i % len(caches)]
                c.decode_step(new_k[i % pool], new_v[i % pool], qs[i % pool], out, ws, stream=cap2)
                gs_bytes += decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads)
    stream.wait_stream(cap2)
    step_graph.replay()
    torch.cuda.synchronize()
    g_reps = max(2, steps // g_steps)
    start.record(stream)
    for _ in range(g_reps):
        step_graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    gstep_ms = start.elapsed_time(end) / (g_reps * g_steps)

    log(f"{flush_steps} steps with {flushes} flushes: {flush_ms*1e3:.2f} us per step")
    log(f"{g_steps} steps captured in one HIP graph: {gstep_ms*1e3:.2f} us per step (replayed)")
    log(f"wall {wall:.3f}s for {steps} steps; {ms_step*1e3:.2f} us per step "
        f"({two_call_ms*1e3:.2f} us as append + decode_attn); decode call "
        f"{dec_ms*1e3:.2f} us (graph replay), {eager_ms*1e3:.2f} us (eager back to back)")
    res = {
        "metric": "decode-attn effective KV GB/s (% of HBM peak) + us/step, Llama-3-8B shape int4",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 3),
        "us_per_step_two_calls": round(two_call_ms * 1e3, 3),
        "us_per_step_with_flushes": round(flush_ms * 1e3, 3),
        "us_per_step_graph": round(gstep_ms * 1e3, 3),
        "gbs_per_step_graph": round(gs_bytes / g_steps / (gstep_ms * 1e-3) / 1e9, 2),
        "steps_with_flushes": {"steps": flush_steps, "flushes": int(flushes),
                               "gbs": round(f_bytes / flush_steps / (flush_ms * 1e-3) / 1e9, 2)},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 MFMA (i32 acc) + f32 softmax", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "context": w.prefill,
                   "codes": f"int{w.code_bits}", "residual": w.residual, "group": w.group,
                   "caches_rotated": args.caches, "parallelism": "single-gpu"},
        "decode_call_us": round(dec_ms * 1e3, 3),
        "decode_call_us_eager": round(eager_ms * 1e3, 3),
        "decode_bytes_per_step": int(bytes_step),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": DECODE_CALL_TRAFFIC,
                     "kernel": "kvq_decode_attn = decode_i8_kernel<128,4,4> (splits merged in-kernel)"},
    }
    return res, (cfg, w)


def run_decode_paths(args, log):
    """Read path (i) against the fused one on the Llama-3-8B int4 decode shape
    ("KV Cache quantization and compression", section 06): restore the whole
    quantized history into a dense bf16 buffer in HBM (kvq_restore), copy the
    window after it, and attend over the dense history (kvq_decode_attn on a
    cache whose window holds every token), against kvq_decode_attn on the
    quantized cache."""
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import KVCache, make_config

    w = ks.LLAMA3_DECODE
    n_caches = args.caches
    cfg, caches = build_caches(w, n_caches, w.prefill + 64, log)
    total = caches[0].state.total
    nq, nt = caches[0].state.quantized, caches[0].state.tail
    # One dense history (a per-layer temporary of path (i)): every token in the
    # bf16 window, nothing quantized.
    dcfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=64,
                       code_bits=w.code_bits, qmax=w.qmax, residual=total, group=w.group)
    dense = KVCache(dcfg, zero=False)
    dense.state.quantized, dense.state.tail, dense.state.total = 0, total, total
    ring = caches[0].sizes.ring
    slots = torch.tensor([(nq + i) % ring for i in range(nt)], device="cuda")
    s = ks.Stream(w, seed=20_000)
    q = ks.decode_query(s).cuda()
    out_f = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    out_d = torch.empty_like(out_f)
    ws = caches[0].workspace(w.q_heads, 1)
    dws = dense.workspace(w.q_heads, 1)
    stream = torch.cuda.current_stream()
    reps = max(4, args.steps // n_caches)

    def timed(fn):
        for c in caches[:2]:
            fn(c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for c in caches:
                fn(c)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * n_caches)

    def restore(c):
        c.restore(dense.k_tail, dense.v_tail)

    def window(c):
        dense.k_tail[:, :, nq:total] = c.k_tail[:, :, slots]
        dense.v_tail[:, :, nq:total] = c.v_tail[:, :, slots]

    def path_i(c):
        restore(c)
        window(c)
        dense.decode_attn(q, out_d, dws)

    fused_us = timed(lambda c: c.decode_attn(q, out_f, ws))
    restore_us = timed(restore)
    window_us = timed(window)
    dense_us = timed(lambda c: dense.decode_attn(q, out_d, dws))
    path_us = timed(path_i)
    caches[-1].decode_attn(q, out_f, ws)
    path_i(caches[-1])
    torch.cuda.synchronize()
    diff = float((out_f - out_d).abs().max())
    units = w.batch * w.kv_heads
    fused_bytes = decode_bytes(cfg, nq, nt, w.q_heads)
    restored = 2 * units * nq * w.head_dim * 2                 # bf16 keys and values written
    dense_read = 2 * units * total * w.head_dim * 2 + w.batch * w.q_heads * w.head_dim * 2
    path_bytes = (fused_bytes - 2 * units * nt * w.head_dim * 2) + restored + 2 * (2 * units * nt * w.head_dim * 2) + dense_read
    log(f"fused decode {fused_us:.2f} us; restore-to-HBM path {path_us:.2f} us (restore {restore_us:.2f}, "
        f"window copy {window_us:.2f}, dense attention {dense_us:.2f}); max |fused - path| {diff:.2e}")
    return {
        "metric": "decode call time by read path, Llama-3-8B shape int4 (restore to HBM + dense attention vs fused)",
        "value": round(path_us, 3), "unit": "us", "n_gpus": 1, "steps": reps * n_caches, "warmup": 2,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 dense history / int4 fused", "data": "synthetic",
        "config": {"workload": w.name + "_read_paths", "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "context": total,
                   "codes": f"int{w.code_bits}", "caches_rotated": n_caches, "parallelism": "single-gpu"},
        "fused_us": round(fused_us, 3),
        "restore_us": round(restore_us, 3),
        "window_copy_us": round(window_us, 3),
        "dense_attention_us": round(dense_us, 3),
        "max_abs_fused_vs_path": diff,
        "algorithmic_bytes": {"fused": int(fused_bytes), "restore_path": int(path_bytes)},
    }


def same_axis_decode_bytes(cfg, nq: int, nt: int, q_heads: int) -> int:
    """Algorithmic bytes of a decode call over a same-axis cache: codes, one
    fp16 Key and one fp16 Value scale per token and run of 64 channels, tail, q."""
    B, H, D = cfg.batch, cfg.kv_heads, cfg.head_dim
    W = D * cfg.code_bits // 8
    es = 2 if cfg.kv_dtype == 0 else 4
    per_unit = 2 * nq * W + 2 * nq * (D // 64) * 2 + 2 * nt * D * es
    return B * H * per_unit + B * q_heads * D * es


def _graph_call_us(calls, replays, stream):
    """Average time of one call of `calls` (one per cache), captured once into a
    HIP graph and replayed back to back between one HIP event pair."""
    import torch
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for fn in calls:
                fn(cap)
    stream.wait_stream(cap)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * len(calls))


def run_axis_ab(args, log):
    """KIVI (Keys per channel over a segment, Values per token) against
    same-axis scales (Keys and Values per token, one scale per run of 64
    channels) -- "KV Cache Quantization Strategies", Step 2 table and
    section 5.1.

    1. The decode call at the Llama-3-8B int4 shape (4096 tokens, 16 caches
       rotated, graph replays): KIVI on the matrix-core kernel, KIVI on the
       vector-ALU kernel, same-axis on the vector-ALU kernel; time and
       algorithmic bytes per call, and each scheme's 4096-token prefill flush.
    2. The error at the video cache's shape (432000 tokens, int2, 8 KV heads):
       single-query decode attention over each quantized cache against exact
       fp32 attention over the unquantized bf16 K/V, for 8 seeded queries.
    """
    import torch

    import kvq_synth as ks
    import quantized_kv_cache_kvq_amd as kvq

    w = ks.LLAMA3_DECODE
    stream = torch.cuda.current_stream()
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    variants = (("kivi_mfma", kvq.KVQ_KIVI, kvq.KVQ_KERNEL_AUTO),
                ("kivi_valu", kvq.KVQ_KIVI, kvq.KVQ_KERNEL_VALU),
                ("same_axis_valu", kvq.KVQ_SAME_AXIS, kvq.KVQ_KERNEL_VALU))
    decode = {}
    for name, scheme, kernel in variants:
        cfg = kvq.make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=w.prefill + 64,
                              code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group,
                              scheme=scheme, decode_kernel=kernel)
        caches, qs, flush_ms = [], [], []
        for i in range(args.caches):
            k, v = ks.device_kv_pair(w, w.prefill, seed=i)
            c = kvq.KVCache(cfg, zero=False)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            c.append(k, v)
            e1.record(stream)
            torch.cuda.synchronize()
            flush_ms.append(e0.elapsed_time(e1))
            del k, v
            caches.append(c)
            qs.append(ks.device_queries(w, seed=i))
        ws = caches[0].workspace(w.q_heads)
        us = _graph_call_us([(lambda st, c=c, q=q: c.decode_attn(q, out, ws, stream=st)) for c, q in zip(caches, qs)],
                            max(4, args.steps // args.caches), stream)
        st = caches[0].state
        nbytes = (same_axis_decode_bytes if scheme == kvq.KVQ_SAME_AXIS else decode_bytes)(cfg, st.quantized, st.tail,
                                                                                          w.q_heads)
        flush_ms.sort()
        decode[name] = {"us_per_call": round(us, 3), "bytes_per_call": int(nbytes),
                        "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "prefill_append_us": round(flush_ms[len(flush_ms) // 2] * 1e3, 1)}
        log(f"{name}: {us:.2f} us per decode call, {nbytes / 1e6:.2f} MB, prefill append "
            f"{flush_ms[len(flush_ms) // 2] * 1e3:.1f} us")
        del caches, qs
        torch.cuda.empty_cache()

    # attention error at the video cache's shape
    wv = ks.VIDEO_BLOCK
    k, v = ks.device_kv_pair(wv, wv.prefill, seed=0)
    sigma = 1.0 / math.sqrt(wv.head_dim)
    g = wv.q_heads // wv.kv_heads
    queries = [ks.device_queries(wv, seed=100 + i) for i in range(8)]
    exact = []
    for q in queries:
        o = torch.empty(wv.batch, wv.q_heads, wv.head_dim, device="cuda")
        for h in range(wv.kv_heads):
            K = k[0, h].float()
            p = torch.softmax((q[0, h * g:(h + 1) * g].float() @ K.T) * sigma, dim=-1)
            o[0, h * g:(h + 1) * g] = p @ v[0, h].float()
        exact.append(o)
    errors = {}
    vout = torch.empty(wv.batch, wv.q_heads, wv.head_dim, device="cuda")
    for name, scheme in (("kivi", kvq.KVQ_KIVI), ("same_axis", kvq.KVQ_SAME_AXIS)):
        cfg = kvq.make_config(batch=wv.batch, kv_heads=wv.kv_heads, head_dim=wv.head_dim, capacity=wv.prefill + 128,
                              code_bits=wv.code_bits, qmax=wv.qmax, residual=wv.residual, group=wv.group,
                              scheme=scheme)
        c = kvq.KVCache(cfg, zero=False)
        c.append(k, v)
        ws = c.workspace(wv.q_heads)
        mx, sq, n = 0.0, 0.0, 0
        for q, ref in zip(queries, exact):
            c.decode_attn(q, vout, ws)
            d = (vout - ref).double()
            mx = max(mx, float(d.abs().max()))
            sq += float((d * d).sum())
            n += d.numel()
        ref_rms = math.sqrt(sum(float((r.double() ** 2).sum()) for r in exact) / n)
        errors[name] = {"attn_max_abs": round(mx, 5), "attn_rms": round(math.sqrt(sq / n), 6),
                        "exact_output_rms": round(ref_rms, 6)}
        log(f"int2 video shape, {name}: attention max-abs {mx:.4f}, RMS {math.sqrt(sq / n):.5f} "
            f"(exact output RMS {ref_rms:.5f})")
        del c, ws
        torch.cuda.empty_cache()
    kivi, sa = decode["kivi_mfma"], decode["same_axis_valu"]
    return {
        "metric": "decode call time, KIVI vs same-axis scales, Llama-3-8B shape int4",
        "value": sa["us_per_call"], "unit": "us", "n_gpus": 1, "steps": max(4, args.steps // args.caches) * args.caches,
        "warmup": 2, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 MFMA or f32 VALU", "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": "llama3_8b_decode_b8_ctx4096_int4_axis_ab", "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "context": w.prefill, "codes": "int4",
                   "same_axis_run": 64, "caches_rotated": args.caches, "parallelism": "single-gpu",
                   "error_workload": wv.name, "error_queries": len(queries)},
        "decode": decode,
        "int2_video_shape_error": errors,
        "same_axis_over_kivi_bytes": round(sa["bytes_per_call"] / kivi["bytes_per_call"], 4),
    }


def paged_decode_bytes(cfg, states, q_heads: int) -> int:
    """Algorithmic bytes of one paged decode call: each sequence's codes,
    scales and window at its own length, plus the queries."""
    H, D = cfg.kv_heads, cfg.head_dim
    W = D * cfg.code_bits // 8
    es = 2 if cfg.kv_dtype == 0 else 4
    total = 0
    for st in states:
        nq, nt = st.quantized, st.tail
        total += H * (2 * nq * W + nq * 2 + (nq // cfg.group) * D * 2 + 2 * nt * D * es)
    return total + cfg.batch * q_heads * D * es


def run_paged_decode(args, log):
    """Decode over paged caches (block table + per-sequence lengths) on the
    Llama-3-8B int4 shape: ragged lengths, and all sequences at 4096 beside
    the uniform cache's decode for the cost of paging."""
    import numpy as np
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import PagedKVCache, make_config

    w = ks.LLAMA3_DECODE
    n_caches = args.caches
    ragged = [int(x) for x in np.random.default_rng(4096).integers(256, 7937, size=w.batch)]
    stream = torch.cuda.current_stream()
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")

    def build(lengths, seed0):
        stride = max(lengths) // 64 + 4
        cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=stride * 64,
                          code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
        caches, qs = [], []
        for i in range(n_caches):
            n_pages = w.batch * stride + 8
            perm = np.random.default_rng(seed0 + i).permutation(n_pages)[:w.batch * stride]
            table = torch.from_numpy(perm.reshape(w.batch, stride).astype(np.int32)).cuda()
            c = PagedKVCache(cfg, n_pages, table)
            k, v = ks.device_kv_pair(w, max(lengths), seed=seed0 + i)
            c.append(k, v, lengths)
            del k, v
            caches.append(c)
            qs.append(ks.device_queries(w, seed=seed0 + i))
        torch.cuda.synchronize()
        return cfg, caches, qs

    def graph_time(calls):
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for fn in calls:
                    fn(cap)
        stream.wait_stream(cap)
        replays = max(2, args.steps // len(calls))
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * len(calls)), replays * len(calls)

    results = {}
    for name, lengths in (("ragged", ragged), ("uniform", [w.prefill] * w.batch)):
        cfg, caches, qs = build(lengths, 30_000 if name == "ragged" else 40_000)
        ws = caches[0].workspace(w.q_heads)
        calls = [(lambda st, c=c, q=q: c.decode_attn(q, out, ws, stream=st)) for c, q in zip(caches, qs)]
        us, n = graph_time(calls)
        nbytes = paged_decode_bytes(cfg, caches[0].states, w.q_heads)
        results[name] = (us, nbytes, n)
        log(f"paged decode ({name} {lengths}): {us:.2f} us per call, {nbytes / (us * 1e-6) / 1e9:.0f} GB/s")
        if name == "ragged":
            # Decode steps (append one token to every sequence, attend with it
            # visible), eager, rotating over the caches: one
            # kvq_paged_decode_step per step, then the same as two calls.
            s = ks.Stream(w, seed=60_000)
            nk, nv = (t.cuda() for t in ks.kv_pair(s, 1))
            ones = [1] * w.batch
            for i in range(2 * len(caches)):
                caches[i % len(caches)].decode_step(nk, nv, ones, qs[i % len(caches)], out, ws)
            steps_k = args.steps
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps_k):
                caches[i % len(caches)].decode_step(nk, nv, ones, qs[i % len(caches)], out, ws)
            e1.record(stream)
            torch.cuda.synchronize()
            step_us = e0.elapsed_time(e1) * 1e3 / steps_k
            e0.record(stream)
            for i in range(steps_k):
                c = caches[i % len(caches)]
                c.append(nk, nv, ones)
                c.decode_attn(qs[i % len(caches)], out, ws)
            e1.record(stream)
            torch.cuda.synchronize()
            two_us = e0.elapsed_time(e1) * 1e3 / steps_k
            results["step"] = (step_us, two_us)
            log(f"paged decode step (ragged): {step_us:.2f} us, {two_us:.2f} us as append + decode")
        del caches, qs
        torch.cuda.empty_cache()
    # the uniform cache at the same shape (matrix-core decode kernel)
    cfg, dense = build_caches(w, n_caches, w.prefill + 64, log)
    dq = [ks.device_queries(w, seed=50_000 + i) for i in range(n_caches)]
    dws = dense[0].workspace(w.q_heads, 1)
    dense_us, _ = graph_time([(lambda st, c=c, q=q: c.decode_attn(q, out, dws, stream=st))
                              for c, q in zip(dense, dq)])
    us, nbytes, n = results["ragged"]
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"uniform cache decode {dense_us:.2f} us per call")
    return {
        "metric": "paged decode-attn effective KV GB/s, Llama-3-8B shape int4, ragged lengths",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": 2,
        "ms_per_step": round(us * 1e-3, 5), "us_per_call": round(us, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 MFMA (i32 acc) + f32 softmax", "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": "llama3_8b_paged_decode_b8_ragged_int4", "batch": w.batch,
                   "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                   "lengths": ragged, "page_tokens": 64, "codes": f"int{w.code_bits}",
                   "caches_rotated": n_caches, "parallelism": "single-gpu"},
        "bytes_per_call": int(nbytes),
        "uniform_4096_paged_us": round(results["uniform"][0], 3),
        "uniform_4096_paged_gbs": round(results["uniform"][1] / (results["uniform"][0] * 1e-6) / 1e9, 2),
        "uniform_4096_unpaged_us": round(dense_us, 3),
        "ragged_step_us": round(results["step"][0], 3),
        "ragged_step_us_two_calls": round(results["step"][1], 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": PAGED_CALL_TRAFFIC,
                     "kernel": "kvq_paged_decode_attn = decode_i8_kernel<128,4,4,paged> (splits merged in-kernel)"},
    }


def block_flops(nq_total: int, tq: int, q_heads: int, head_dim: int, batch: int = 1,
                frame_tokens: int = 1) -> float:
    """Algorithmic FLOPs of one block: QK^T and PV over N cached tokens plus the
    block's own visible tokens (query i sees those up to the end of its frame
    of frame_tokens positions, clipped to the block; i + 1 of them for 1)."""
    own = 0
    for i in range(tq):
        own += min(tq, ((nq_total + i) // frame_tokens + 1) * frame_tokens - nq_total)
    pairs = tq * nq_total + own
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
    F = args.frame_tokens
    for _ in range(warmup):
        c.block_attn(q, kb, vb, out, ws, frame_tokens=F)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        c.block_attn(q, kb, vb, out, ws, frame_tokens=F)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = block_flops(c.state.total, w.block_q, w.q_heads, w.head_dim, w.batch, F)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"video block (frames of {F}): {ms:.3f} ms per block, {tflops:.1f} TFLOP/s")
    return {
        "metric": ("causal block attention over the quantized cache, ms per block" if F == 1 else
                   "frame-causal block attention over the quantized cache, ms per block"),
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/f16 MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "cached": c.state.total,
                   "block_q": w.block_q, "frame_tokens": F, "codes": f"int{w.code_bits}",
                   "parallelism": "single-gpu"},
        "flops_per_block": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4), "traffic": BLOCK_CALL_TRAFFIC,
                     "kernel": "kvq_block_attn = block_kernel<128,2> + block_merge_kernel<128>"},
    }


def run_paged_block(args, log):
    """The video block (1024 causal queries, 432000-token int2 cache) with the
    cache in 64-token pages behind a shuffled block table, timed beside the
    same block on the uniform cache."""
    import numpy as np
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import KVCache, PagedKVCache, make_config

    w = ks.VIDEO_BLOCK
    cap = w.prefill + 128
    stride = (cap + 63) // 64
    cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=stride * 64,
                      code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
    s = ks.Stream(w, seed=0)
    k, v = (t.cuda() for t in ks.kv_pair(s, w.prefill))
    c = KVCache(cfg, zero=False)
    c.append(k, v)
    n_pages = w.batch * stride + 16
    perm = np.random.default_rng(432000).permutation(n_pages)[:w.batch * stride]
    pc = PagedKVCache(cfg, n_pages, torch.from_numpy(perm.reshape(w.batch, stride).astype(np.int32)).cuda())
    pc.append(k, v, [w.prefill] * w.batch)
    del k, v
    q, kb, vb = (t.cuda() for t in ks.block_inputs(s, w.block_q))
    out = torch.empty(w.batch, w.block_q, w.q_heads, w.head_dim, device="cuda")
    ws = c.workspace(w.q_heads, w.block_q)
    stream = torch.cuda.current_stream()
    steps, warmup = max(1, args.steps // 20), max(1, args.warmup // 10)
    F = args.frame_tokens

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / steps

    paged_ms = timed(lambda: pc.block_attn(q, kb, vb, out, ws, frame_tokens=F))
    dense_ms = timed(lambda: c.block_attn(q, kb, vb, out, ws, frame_tokens=F))
    flops = block_flops(c.state.total, w.block_q, w.q_heads, w.head_dim, w.batch, F)
    tflops = flops / (paged_ms * 1e-3) / 1e12
    log(f"paged video block: {paged_ms:.3f} ms ({tflops:.1f} TFLOP/s); uniform cache {dense_ms:.3f} ms")
    return {
        "metric": "block attention over a paged quantized cache, ms per block",
        "value": round(paged_ms, 4), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/f16 MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name + "_paged", "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "cached": c.state.total,
                   "block_q": w.block_q, "frame_tokens": F, "codes": f"int{w.code_bits}", "page_tokens": 64,
                   "parallelism": "single-gpu"},
        "uniform_cache_ms": round(dense_ms, 4),
        "flops_per_block": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": PAGED_BLOCK_CALL_TRAFFIC,
                     "kernel": "kvq_paged_block_attn = block_kernel<128,2,PagedBlock> + block_merge_kernel<128>"},
    }


def run_long_decode(args, log):
    """One step = 32 sequential decode calls, one per layer cache of 131072 tokens."""
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import KVCache, make_config

    w = ks.LONG_CONTEXT
    cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim,
                      capacity=w.prefill + 256, code_bits=w.code_bits, qmax=w.qmax,
                      residual=w.residual, group=w.group)
    caches, qs = [], []
    for layer in range(w.layers):
        k, v = ks.device_kv_pair(w, w.prefill, seed=layer)
        c = KVCache(cfg, zero=False)
        c.append(k, v)
        del k, v
        caches.append(c)
        qs.append(ks.device_queries(w, seed=layer))
    torch.cuda.synchronize()
    log(f"built {w.layers} layer caches of {w.prefill} tokens")
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    ws = caches[0].workspace(w.q_heads, 1)
    stream = torch.cuda.current_stream()
    steps, warmup = max(2, args.steps // 20), max(1, args.warmup // 10)

    def step():
        for layer, c in enumerate(caches):
            c.decode_attn(qs[layer], out, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = sum(decode_bytes(cfg, c.state.quantized, c.state.tail, w.q_heads) for c in caches)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"long decode: {ms * 1e3:.1f} us per 32-layer step, {gbs:.0f} GB/s")
    return {
        "metric": "decode-attn effective KV GB/s, 32 layers of 131072 tokens, int4",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 MFMA (i32 acc) + f32 softmax", "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "context": w.prefill, "layers": w.layers,
                   "codes": f"int{w.code_bits}", "parallelism": "single-gpu"},
        "bytes_per_step": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": LONG_CALL_TRAFFIC,
                     "kernel": "kvq_decode_attn = decode_i8_kernel<128,4,4> (splits merged in-kernel)"},
    }


def append_bytes(cfg, st0, st1, n_new: int) -> int:
    """Algorithmic bytes of one append: new tokens read, surviving tokens written to
    the tail ring, flushed tokens read (old tail + new) and their codes and scales
    written."""
    units = cfg.batch * cfg.kv_heads
    D, es = cfg.head_dim, 2 if cfg.kv_dtype == 0 else 4
    W = D * cfg.code_bits // 8
    flushed = st1.quantized - st0.quantized
    kept_new = n_new - max(0, flushed - st0.tail)
    nseg = st1.segments - st0.segments
    per_unit = 2 * n_new * D * es                  # read K, V of the new tokens
    per_unit += 2 * kept_new * D * es              # write them to the tail ring
    per_unit += 2 * min(flushed, st0.tail) * D * es  # read the flushed tokens that sat in the tail
    per_unit += 2 * flushed * W + flushed * 2 + nseg * D * 2   # codes, V scales, K scales
    return units * per_unit


def run_append(args, log, bits: int):
    """128 appends of 16 tokens into 4096-token caches of 16 x 8 heads.

    The 128 calls are captured once into a HIP graph (the host-side token
    accounting runs at capture) and the graph is replayed: the replays time
    the GPU work of the whole run without per-call host overhead.  Replays
    rewrite the same buffers, so only the first pass leaves the exact cache
    the calls describe; the timing does not depend on the values.  The eager
    (host-driven) time per append is reported beside it.
    """
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import KVCache, make_config

    w = ks.APPEND_INT8 if bits == 8 else ks.APPEND_INT4
    total = w.prefill + w.steps * w.step_tokens
    cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=total,
                      code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
    k0, v0 = ks.device_kv_pair(w, w.prefill, seed=0)
    kn, vn = ks.device_kv_pair(w, w.steps * w.step_tokens, seed=1)
    chunks = [(kn[:, :, i * w.step_tokens:(i + 1) * w.step_tokens].contiguous(),
               vn[:, :, i * w.step_tokens:(i + 1) * w.step_tokens].contiguous()) for i in range(w.steps)]

    def fresh():
        c = KVCache(cfg, zero=False)
        c.append(k0, v0)
        torch.cuda.synchronize()
        return c

    def snap(st):
        return type("S", (), dict(quantized=st.quantized, tail=st.tail, total=st.total,
                                  flushed_last=st.flushed_last, segments=st.segments))

    # eager: host-driven calls, one event pair around the run
    stream = torch.cuda.current_stream()
    eager_ms = []
    for r in range(2):
        c = fresh()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for kc, vc in chunks:
            c.append(kc, vc, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_ms.append(e0.elapsed_time(e1))
    # graph: capture the 128 calls once, replay
    c = fresh()
    graph = torch.cuda.CUDAGraph()
    nbytes, nflush = 0, 0
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for kc, vc in chunks:
                st0 = snap(c.state)
                c.append(kc, vc, cap)
                nbytes += append_bytes(cfg, st0, c.state, w.step_tokens)
                nflush += int(c.state.flushed_last > 0)
    stream.wait_stream(cap)
    runs = max(3, args.steps // 20)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(runs):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / runs
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"append int{bits}: graph {ms * 1e3:.1f} us per {w.steps} appends ({nflush} with a flush), "
        f"{gbs:.0f} GB/s; eager {min(eager_ms) * 1e3 / w.steps:.1f} us per append")
    return {
        "metric": f"append/quantize write path GB/s, int{bits}",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": w.steps, "warmup": 2,
        "ms_per_step": round(ms / w.steps, 5), "us_per_append": round(ms * 1e3 / w.steps, 3),
        "us_per_append_eager": round(min(eager_ms) * 1e3 / w.steps, 3), "flushes_per_run": nflush,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, f32 scale arithmetic, int codes", "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": w.name, "batch": w.batch, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                   "prefill": w.prefill, "appends": w.steps, "tokens_per_append": w.step_tokens,
                   "codes": f"int{bits}", "residual": w.residual, "group": w.group,
                   "parallelism": "single-gpu", "timing": "HIP graph of the 128 appends, replayed"},
        "bytes_per_run": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": APPEND_RUN_TRAFFIC[bits],
                     "kernel": f"kvq_append = flush_kernel<{bits}> + tail_kernel"},
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_decode_case():
    """The oracle's state and query for the Llama-3-8B int4 decode workload."""
    import kvq_synth as ks
    from oracle.cache import KVQuantizationStrategies

    w = ks.LLAMA3_DECODE
    s = ks.Stream(w, seed=0)
    k, v = ks.kv_pair(s, w.prefill)
    o = KVQuantizationStrategies(qmax=w.qmax, scale_storage="fp16", group=w.group)
    st = o.append_and_partition(None, k.float().numpy(), v.float().numpy(), w.residual)
    q = ks.decode_query(s).float().numpy()
    return w, st, q


def _oracle_units_worker(units, budget_s):
    """One process's share of the decode call: the oracle over its (batch,
    KV head) units, repeated for about budget_s seconds, one thread."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt
    w, st, q = _oracle_decode_case()
    sigma = 1.0 / math.sqrt(w.head_dim)
    with threadpool_limits(limits=1):
        oatt.decode_attention(st, q, sigma, units=units)      # warm
        reps, t = 0, time.perf_counter()
        while True:
            oatt.decode_attention(st, q, sigma, units=units)
            reps += 1
            if time.perf_counter() - t >= budget_s:
                break
    return reps, time.perf_counter() - t


def cpu_baseline_decode(budget_s: float, log):
    """The CPU oracle's decode attention on the Llama-3-8B int4 workload:
    whole calls (all 64 (batch, KV head) units) on one thread, then the same
    units split over one process per host core (the per-process call time is
    the slowest share's).  Runs before the GPU is touched."""
    import concurrent.futures
    import multiprocessing

    from quantized_kv_cache_kvq_amd import make_config

    w, st, q = _oracle_decode_case()
    cfg = make_config(batch=1, kv_heads=1, head_dim=w.head_dim, capacity=w.prefill,
                      code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
    nq, nt = st["quantized_tokens"], st["key_residual"].shape[-2]
    unit_bytes = decode_bytes(cfg, nq, nt, w.q_heads // w.kv_heads)
    units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    call_bytes = len(units) * unit_bytes
    reps1, dt1 = _oracle_units_worker(units, budget_s / 2)
    one = call_bytes * reps1 / dt1 / 1e9
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    n = max(1, min(16, ncpu, len(units)))
    shares = [units[i::n] for i in range(n)]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=n, mp_context=ctx) as ex:
        res = list(ex.map(_oracle_units_worker, shares, [budget_s / 2] * n))
    per_call = max(dt / reps for reps, dt in res)      # the slowest share sets the call
    alln = call_bytes / per_call / 1e9
    log(f"cpu oracle: {dt1 / reps1 * 1e3:.1f} ms per call on 1 thread, {per_call * 1e3:.1f} ms on {n} processes")
    return {"value": round(alln, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"full fp64 decode-attention calls (restore + softmax over all {len(units)} "
                      f"(batch, KV head) units) of the Llama-3-8B int4 workload at {w.prefill} tokens: "
                      f"{per_call * 1e3:.1f} ms per call with the units split over {n} single-thread "
                      f"processes (the slowest share's time, {budget_s / 2:.0f} s each), "
                      f"{dt1 / reps1 * 1e3:.1f} ms per call on one thread ({reps1} calls)",
            "value_1thread": round(one, 4), "ms_per_call": round(per_call * 1e3, 2),
            "ms_per_call_1thread": round(dt1 / reps1 * 1e3, 2),
            "cpu": _cpu_model(), "nproc": os.cpu_count()}


def run_hbm_copy(args, log):
    """A plain device-to-device copy of 256 MiB (the runtime's copy kernel),
    ten times back to back: a reference read+write rate for this box, and a
    kernel of known size for scaling the HBM traffic counters."""
    import torch

    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    log(f"hbm copy: {ms * 1e3:.1f} us per 256 MiB copy, {gbs:.0f} GB/s read + write")
    return {"metric": "device copy GB/s (read + write)", "value": round(gbs, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": reps, "warmup": 1, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": {"workload": "hbm_copy_256MiB", "bytes": nbytes}}


def _graph_us(launches, replays: int, log=None) -> float:
    """Average µs of one launch: the launches captured once into a HIP graph
    on a side stream, the graph replayed back to back, one HIP event pair on
    the current stream around the replays."""
    import torch

    stream = torch.cuda.current_stream()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for fn in launches:
                fn(cap)
    stream.wait_stream(cap)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * len(launches))


def run_hbm_read(args, log):
    """Read-only HBM stream with the probe kernel (128-bit loads, one word
    stored per workgroup): at the decode call's size, rotating over 16
    buffers so that nothing is served from the 256 MB Infinity Cache, and at
    1 GiB; swept over workgroup counts and loads in flight per thread.  An
    empty kernel gives the launch floor."""
    import torch

    import kvq_synth as ks
    from quantized_kv_cache_kvq_amd import make_config, probes

    probes.load()
    w = ks.LLAMA3_DECODE
    cfg = make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=w.prefill,
                      code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group)
    dec = decode_bytes(cfg, w.prefill - w.residual, w.residual, w.q_heads)
    dec = (dec + 15) // 16 * 16
    n_buf = 16
    bufs = [torch.ones(dec // 4, dtype=torch.int32, device="cuda") for _ in range(n_buf)]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    reps = max(4, args.steps // 10)
    small = {}
    for wgs in (256, 512, 1024, 2048, 4096):
        for depth in (1, 2, 4, 8, 16):
            us = _graph_us([(lambda st, b=b: probes.stream_read(b, wgs, depth, sink, st)) for b in bufs], reps)
            small[f"{wgs}x{depth}"] = round(us, 3)
            log(f"hbm read {dec} B, {wgs} workgroups, depth {depth}: {us:.2f} us, {dec / us / 1e3:.0f} GB/s")
    del bufs
    torch.cuda.empty_cache()
    # The input of one 128-token flush of the append workload (16 x 8 heads,
    # K and V, bf16): 8,388,608 bytes, 40 buffers rotated (335 MB).
    fl = ks.APPEND_INT4
    fbytes = fl.batch * fl.kv_heads * fl.group * fl.head_dim * 2 * 2
    fbufs = [torch.ones(fbytes // 4, dtype=torch.int32, device="cuda") for _ in range(40)]
    flush = {}
    for wgs in (256, 512, 1024, 2048):
        for depth in (2, 4, 8, 16):
            us = _graph_us([(lambda st, b=b: probes.stream_read(b, wgs, depth, sink, st)) for b in fbufs], reps)
            flush[f"{wgs}x{depth}"] = round(us, 3)
            log(f"hbm read {fbytes} B, {wgs} workgroups, depth {depth}: {us:.2f} us, {fbytes / us / 1e3:.0f} GB/s")
    del fbufs
    torch.cuda.empty_cache()
    best_flush = min(flush.items(), key=lambda kv: kv[1])
    big_bytes = 1 << 30
    big = torch.ones(big_bytes // 4, dtype=torch.int32, device="cuda")
    large = {}
    for wgs in (512, 1024, 2048, 4096, 8192, 16384):
        for depth in (4, 8, 16):
            us = _graph_us([(lambda st: probes.stream_read(big, wgs, depth, sink, st))], max(4, reps // 4))
            large[f"{wgs}x{depth}"] = round(us, 2)
            log(f"hbm read 1 GiB, {wgs} workgroups, depth {depth}: {us:.1f} us, {big_bytes / us / 1e3:.0f} GB/s")
    del big
    empty = {}
    for wgs in (512, 2048):
        empty[str(wgs)] = round(_graph_us([(lambda st: probes.empty(wgs, st))] * 16, reps), 3)
        log(f"empty kernel, {wgs} workgroups: {empty[str(wgs)]:.2f} us per launch")
    best_small = min(small.items(), key=lambda kv: kv[1])
    best_large = min(large.items(), key=lambda kv: kv[1])
    at512 = min((v, k) for k, v in small.items() if k.startswith("512x"))
    return {
        "metric": "read-only HBM stream GB/s (probe kernel)",
        "value": round(big_bytes / best_large[1] / 1e3, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": reps, "warmup": 2, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32x4 loads", "data": "synthetic",
        "config": {"workload": "hbm_read_stream", "small_bytes": dec, "small_buffers": n_buf,
                   "large_bytes": big_bytes},
        "small_best_us": best_small[1], "small_best_shape": best_small[0],
        "small_best_gbs": round(dec / best_small[1] / 1e3, 2),
        "small_512wg_us": at512[0], "small_512wg_shape": at512[1],
        "small_512wg_gbs": round(dec / at512[0] / 1e3, 2),
        "large_best_shape": best_large[0],
        "flush_input_bytes": fbytes, "flush_input_best_us": best_flush[1], "flush_input_best_shape": best_flush[0],
        "small_us_by_shape": small, "large_us_by_shape": large, "flush_input_us_by_shape": flush,
        "empty_kernel_us": empty,
        "roofline": {"bound": "hbm", "achieved": round(big_bytes / best_large[1] / 1e3, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(big_bytes / best_large[1] / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "stream_read_kernel"},
    }


def run_mfma_peak(args, log):
    """Matrix-core throughput of the probe loop (eight independent chains per
    wave, register operands), per instruction kind, at one, two and four waves
    per SIMD."""
    import torch

    from quantized_kv_cache_kvq_amd import probes

    probes.load()
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    iters = 4000
    res = {}
    for kind, (name, ops) in probes.MFMA_KINDS.items():
        for wgs in (256, 512, 1024):
            for _ in range(2):
                probes.mfma(kind, wgs, iters, sink)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 5
            e0.record(stream)
            for _ in range(n):
                probes.mfma(kind, wgs, iters, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            work = wgs * 4 * iters * 8 * ops
            tf = work / (ms * 1e-3) / 1e12
            res[f"{name}@{wgs}"] = round(tf, 1)
            log(f"{name}, {wgs} workgroups: {ms:.3f} ms, {tf:.0f} T(FL)OP/s")
    bf16 = max(v for k, v in res.items() if "bf16" in k)
    return {
        "metric": "matrix-core throughput, probe loop (TFLOP/s; i8 in TOP/s)",
        "value": bf16, "unit": "TFLOP/s", "n_gpus": 1, "steps": 5, "warmup": 2,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 / f16 / i8",
        "data": "synthetic", "config": {"workload": "mfma_peak", "iters": iters},
        "by_kind": res,
        "roofline": {"bound": "mfma", "achieved": bf16, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(bf16 / 2500.0, 4), "traffic": None, "kernel": "mfma_kernel<bf16>"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--caches", type=int, default=16)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--frame-tokens", type=int, default=1,
                    help="video_block: frame length of the block mask (1 = token-causal)")
    ap.add_argument("--workload", choices=["llama3_decode", "video_block", "long_decode", "append_int8",
                                           "append_int4", "hbm_copy", "decode_paths", "paged_decode", "paged_block",
                                           "hbm_read", "mfma_peak", "axis_ab"],
                    default="llama3_decode",
                    help="llama3_decode (default): the append + decode step; video_block: one "
                         "1024-query causal block against the 432000-token int2 cache; long_decode: "
                         "32 layers of 131072-token caches; append_int8/int4: 128 appends of 16 "
                         "tokens into 4096-token caches (16 x 8 heads); hbm_copy: a plain 256 MiB "
                         "device copy (reference rate, and the known-size kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters); decode_paths: the decode call by "
                         "restore-to-HBM + dense attention against the fused kernel; paged_decode: "
                         "decode over paged caches (block table, ragged per-sequence lengths); paged_block: "
                         "the video block over a paged cache, beside the uniform cache; hbm_read: the "
                         "read-only stream probe swept over workgroups and loads in flight; mfma_peak: "
                         "the matrix-core probe loop per instruction kind; axis_ab: KIVI against "
                         "same-axis scales (decode time and bytes at the Llama-3-8B shape, and the int2 "
                         "attention error at the video cache's shape)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cpu = None
    if args.workload == "llama3_decode" and not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(args.cpu_budget, log)      # before anything touches the GPU
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import quantized_kv_cache_kvq_amd as kvq
    if not os.path.exists(kvq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    kvq.load()
    if args.workload == "hbm_copy":
        res = run_hbm_copy(args, log)
    elif args.workload == "hbm_read":
        res = run_hbm_read(args, log)
    elif args.workload == "mfma_peak":
        res = run_mfma_peak(args, log)
    elif args.workload == "video_block":
        res = run_video_block(args, log)
    elif args.workload == "long_decode":
        res = run_long_decode(args, log)
    elif args.workload == "decode_paths":
        res = run_decode_paths(args, log)
    elif args.workload == "paged_decode":
        res = run_paged_decode(args, log)
    elif args.workload == "paged_block":
        res = run_paged_block(args, log)
    elif args.workload == "axis_ab":
        res = run_axis_ab(args, log)
    elif args.workload.startswith("append_"):
        res = run_append(args, log, 8 if args.workload == "append_int8" else 4)
    else:
        res, _ = run_decode(args, log)
        if cpu is not None:
            res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
