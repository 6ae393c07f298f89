"""GPU parity of kvq_decode_step: append then attend in one call.

The step must leave the same cache bytes and state as kvq_append followed by
kvq_decode_attn, and its output must match the fp64 oracle (max-abs 2e-3)
and the two-call sequence (float rounding only: the appended tokens enter
the softmax in the merge pass instead of the decode kernel).  The order per
step -- append, then attend with the new token visible -- is that of "KV
Cache quantization and compression", section 02.
"""
import numpy as np
import pytest
import torch

import kvq_synth as ks
import quantized_kv_cache_kvq_amd as kvq
from harness import Pair, f32, max_abs, note

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

TOL = 2e-3
TOL_PAIR = 1e-4       # fused step against append + decode on the same device


def run_steps(w, prefill, steps, n_new=1, num_splits=0, capacity=None, check_every=16):
    fused, split = Pair(w, capacity or prefill + steps * n_new + 64), None
    split = Pair(w, capacity or prefill + steps * n_new + 64)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, prefill)
    fused.append(k, v)
    split.append(k, v)
    worst = worst_pair = 0.0
    flushes = fused_steps = 0
    for i in range(steps):
        k, v = ks.kv_pair(s, n_new)
        q = ks.decode_query(s)
        nxt = kvq.kvq_plan_append(fused.cfg, fused.cache.state, n_new)
        flushes += nxt.flushed_last > 0
        fused_steps += nxt.flushed_last == 0
        got, _ = fused.step(k, v, q, num_splits=num_splits)
        split.append(k, v)
        ref2, _ = split.decode(q, num_splits=num_splits)
        ref = fused.decode_ref(q)
        worst = max(worst, max_abs(got, ref))
        worst_pair = max(worst_pair, max_abs(got, ref2))
        if i % check_every == check_every - 1 or i == steps - 1:
            fused.check_state()
            fused.check_buffers()
    return worst, worst_pair, flushes, fused_steps


@needs_gpu
def test_decode_step_llama_shape_across_a_flush():
    """Llama-3-8B decode shape (reduced batch): 1-token steps through a flush."""
    w = ks.small(ks.LLAMA3_DECODE, batch=2)
    note("decode step llama shape")
    worst, worst_pair, flushes, fused_steps = run_steps(w, prefill=300, steps=100)
    note(f"decode step llama: max-abs {worst:.3e}, vs two calls {worst_pair:.3e}, "
         f"{flushes} flush steps, {fused_steps} single-pass steps")
    assert flushes >= 1 and fused_steps >= 90
    assert worst <= TOL
    assert worst_pair <= TOL_PAIR


@needs_gpu
@pytest.mark.parametrize("n_new,num_splits", [(3, 0), (1, 1), (16, 2), (5, 7), (1, 6)])
def test_decode_step_token_counts_and_splits(n_new, num_splits):
    w = ks.small(ks.LLAMA3_DECODE, batch=1, kv_heads=2, q_heads=8)
    note(f"decode step n_new={n_new} splits={num_splits}")
    worst, worst_pair, flushes, fused_steps = run_steps(w, prefill=300, steps=12, n_new=n_new,
                                                        num_splits=num_splits, check_every=4)
    assert fused_steps >= 1
    assert worst <= TOL
    assert worst_pair <= TOL_PAIR


@needs_gpu
@pytest.mark.parametrize("D,bits,qmax,gqa", [(64, 8, 127, 2), (128, 2, 1, 1), (64, 4, 7, 8), (128, 4, 7, 8)])
def test_decode_step_other_shapes(D, bits, qmax, gqa):
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=2 * gqa, head_dim=D, code_bits=bits,
                 qmax=qmax)
    note(f"decode step D={D} bits={bits} gqa={gqa}")
    worst, worst_pair, _, fused_steps = run_steps(w, prefill=300, steps=10, check_every=5)
    assert fused_steps == 10
    assert worst <= TOL
    assert worst_pair <= TOL_PAIR


@needs_gpu
def test_decode_step_overflow_only_and_empty_cache():
    """Per-append flushes (G = 0) and a first step on an empty cache take the
    two-call path inside the step; results are unchanged."""
    w = ks.small(ks.TINY, batch=2, kv_heads=2, q_heads=4, head_dim=64, code_bits=4, qmax=7,
                 residual=10, group=0, kv_dtype="bf16")
    note("decode step overflow-only")
    worst, worst_pair, flushes, _ = run_steps(w, prefill=0, steps=20, capacity=256, check_every=5)
    assert flushes >= 10
    assert worst <= TOL
    assert worst_pair <= TOL_PAIR


@needs_gpu
def test_decode_step_errors_leave_state_unchanged():
    w = ks.small(ks.LLAMA3_DECODE, batch=1, kv_heads=2, q_heads=8)
    p = Pair(w, 512)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, 100)
    p.append(k, v)
    before = (p.cache.state.quantized, p.cache.state.tail, p.cache.state.total)
    k, v = ks.kv_pair(s, 1)
    q = ks.decode_query(s).cuda()
    out = torch.empty(1, 8, w.head_dim, device="cuda")
    ws = p.cache.workspace(8, 1)
    c = p.cache
    with pytest.raises(kvq.KVQError):      # q_heads not a multiple of kv_heads
        kvq.kvq_decode_step(c.cfg, c.state, c.c, k.cuda(), v.cuda(), 1, q, 7, 0.1, 0, out, ws)
    with pytest.raises(kvq.KVQError):      # workspace too small
        kvq.kvq_decode_step(c.cfg, c.state, c.c, k.cuda(), v.cuda(), 1, q, 8, 0.1, 0, out, ws[:16])
    with pytest.raises(kvq.KVQError):      # capacity exceeded
        big = torch.zeros(1, 2, 1000, w.head_dim, dtype=torch.bfloat16, device="cuda")
        kvq.kvq_decode_step(c.cfg, c.state, c.c, big, big, 1000, q, 8, 0.1, 0, out, ws)
    torch.cuda.synchronize()
    assert (c.state.quantized, c.state.tail, c.state.total) == before
    p.check_buffers()


@needs_gpu
def test_decode_steps_captured_in_one_graph():
    """Twelve decode steps, one of them through a 128-token flush, captured in
    one HIP graph and replayed once: every output and the final cache bytes
    equal those of the same steps run eagerly (bit for bit), and the cache
    matches the oracle's."""
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=8)
    steps = 12
    pairs = []
    for _ in range(2):
        p = Pair(w, 512)
        s = ks.Stream(w, seed=77)
        k, v = ks.kv_pair(s, 380)          # window of 252 tokens: the fourth step flushes
        p.append(k, v)
        pairs.append(p)
    s = ks.Stream(w, seed=78)
    inputs = []
    for _ in range(steps):
        k, v = ks.kv_pair(s, 1)
        inputs.append((k, v, ks.decode_query(s)))
    dev = [(k.cuda(), v.cuda(), q.cuda()) for k, v, q in inputs]
    shape = (w.batch, w.q_heads, w.head_dim)
    # eager
    pe = pairs[0]
    ws_e = pe.cache.workspace(w.q_heads, 1)
    outs_e = [torch.full(shape, float("nan"), device="cuda") for _ in range(steps)]
    for (k, v, q), out in zip(dev, outs_e):
        pe.cache.decode_step(k, v, q, out, ws_e)
    # captured, then replayed once
    pg = pairs[1]
    ws_g = pg.cache.workspace(w.q_heads, 1)
    outs_g = [torch.full(shape, float("nan"), device="cuda") for _ in range(steps)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    note("decode steps graph capture")
    flushed = 0
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for (k, v, q), out in zip(dev, outs_g):
                pg.cache.decode_step(k, v, q, out, ws_g, stream=cap)
                flushed += pg.cache.state.flushed_last
    torch.cuda.current_stream().wait_stream(cap)
    assert flushed == 128
    graph.replay()
    torch.cuda.synchronize()
    for i in range(steps):
        assert torch.equal(outs_g[i], outs_e[i]), i
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "k_tail", "v_tail"):
        assert torch.equal(getattr(pg.cache, name), getattr(pe.cache, name)), name
    for k, v, _ in inputs:
        pg.ost = pg.oracle.append_and_partition(pg.ost, f32(k), f32(v), w.residual)
    pg.check_state()
    pg.check_buffers()
    assert max_abs(outs_g[-1].cpu().numpy(), pg.decode_ref(inputs[-1][2])) <= TOL
