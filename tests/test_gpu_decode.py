"""GPU parity of kvq_decode_attn against the fp64 oracle (max-abs 2e-3).

The oracle attends over the restored codes the oracle itself produced (which
the append tests show are byte-identical to the device's), so the comparison
isolates the attention kernel.
"""
import numpy as np
import pytest
import torch

import kvq_synth as ks
from harness import Pair, max_abs, note

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

TOL = 2e-3


def build(w, n, capacity=None, seed=None):
    p = Pair(w, capacity or (n + 128))
    s = ks.Stream(w, seed)
    k, v = ks.kv_pair(s, n)
    note(f"decode build {w.name} n={n}")
    p.append(k, v)
    return p, s


@needs_gpu
def test_tiny_decode_steps():
    w = ks.TINY
    p, s = build(w, w.prefill, capacity=128)
    ws = p.cache.workspace(w.q_heads)
    for step in range(w.steps):
        k, v = ks.kv_pair(s, 1)
        p.append(k, v)
        q = ks.decode_query(s)
        note(f"tiny decode step {step}")
        got, _ = p.decode(q, ws=ws)
        err = max_abs(got, p.decode_ref(q))
        assert err <= TOL, (step, err)


@needs_gpu
@pytest.mark.parametrize("D,bits,qmax,g", [(128, 4, 7, 4), (128, 8, 127, 4), (128, 2, 1, 4),
                                           (64, 4, 7, 2), (64, 2, 1, 8), (32, 4, 7, 1),
                                           (32, 8, 127, 8), (16, 8, 7, 4), (128, 4, 7, 8),
                                           (128, 4, 7, 1), (128, 4, 7, 2), (64, 4, 7, 1),
                                           (64, 4, 7, 8)])
def test_decode_shapes(D, bits, qmax, g):
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=2 * g, head_dim=D, code_bits=bits,
                 qmax=qmax, residual=128, group=128 if D != 16 else 64)
    p, s = build(w, 1000)         # 768 quantized (6 groups) + 232 tail: ragged tail tiles
    q = ks.decode_query(s)
    got, _ = p.decode(q)
    err = max_abs(got, p.decode_ref(q))
    note(f"decode D={D} bits={bits} g={g}: max-abs {err:.3e}")
    assert err <= TOL


@needs_gpu
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 40, 64, 100, 256])
def test_decode_split_invariance(splits):
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=8)
    p, s = build(w, 1500)
    q = ks.decode_query(s)
    ref = p.decode_ref(q)
    ws = p.cache.workspace(8)
    note(f"decode splits={splits}")
    got, _ = p.decode(q, num_splits=splits, ws=ws)
    assert max_abs(got, ref) <= TOL
    # the arrival counters are left cleared: a second call on it is still right
    torch.cuda.synchronize()
    assert not ws[:64].any()
    got2, _ = p.decode(q, num_splits=splits, ws=ws)
    assert max_abs(got2, ref) <= TOL


@needs_gpu
@pytest.mark.parametrize("n", [1, 2, 63, 64, 127, 128, 129, 255, 256, 257])
def test_decode_edge_lengths(n):
    w = ks.small(ks.LLAMA3_DECODE, batch=1, kv_heads=2, q_heads=8)
    p, s = build(w, n)
    q = ks.decode_query(s)
    got, _ = p.decode(q)
    assert max_abs(got, p.decode_ref(q)) <= TOL


@needs_gpu
def test_decode_overflow_only_segments():
    w = ks.small(ks.TINY, batch=2, kv_heads=2, q_heads=4, head_dim=64, code_bits=4, qmax=7,
                 residual=10, group=0, kv_dtype="bf16")
    p = Pair(w, 512)
    s = ks.Stream(w)
    for n in (100, 1, 7, 64, 3):
        k, v = ks.kv_pair(s, n)
        p.append(k, v)
    q = ks.decode_query(s)
    got, _ = p.decode(q)
    assert max_abs(got, p.decode_ref(q)) <= TOL


@needs_gpu
def test_decode_llama3_full_size():
    """The benchmarked call: batch 8, 32 / 8 heads, 4096 tokens, int4 -- the
    append's codes, scales, window and counters bit-exact, then one decode
    step (append a token, attend) on every (batch, head) against the oracle."""
    w = ks.LLAMA3_DECODE
    p, s = build(w, w.prefill)
    p.check_state()
    p.check_buffers()
    k, v = ks.kv_pair(s, 1)          # decode step: append the new token, then attend
    p.append(k, v)
    p.check_state()
    q = ks.decode_query(s)
    note("decode llama3 full")
    got, ws = p.decode(q)
    ref = p.decode_ref(q)
    err = max_abs(got, ref)
    note(f"decode llama3 full: max-abs {err:.3e}")
    assert err <= TOL, err
    torch.cuda.synchronize()
    assert not ws[:64].any()         # arrival counters back at 0


@needs_gpu
@pytest.mark.parametrize("layer", [0, 31])
def test_decode_long_context_full_layer(layer):
    """One long-context layer in full: 131072 tokens, the layer's own seed
    (layers 0 and 31 of the 32 the benchmark steps through), codes, scales
    and counters bit-exact, and every (KV head, query head) against the
    oracle."""
    w = ks.LONG_CONTEXT
    p, s = build(w, w.prefill, seed=layer)
    p.check_state()
    p.check_buffers()
    q = ks.decode_query(s)
    note(f"decode long context layer {layer}")
    got, _ = p.decode(q)
    ref = p.decode_ref(q)
    err = max_abs(got, ref)
    note(f"decode long context layer {layer}: max-abs {err:.3e}")
    assert not np.isnan(ref).any()
    assert err <= TOL


@needs_gpu
@pytest.mark.parametrize("D,bits,qmax", [(128, 4, 7), (128, 2, 1), (64, 8, 127)])
def test_decode_zero_query_is_mean_of_values(D, bits, qmax):
    """q = 0 gives uniform weights: the output is the mean of the restored values."""
    w = ks.small(ks.LLAMA3_DECODE, batch=1, kv_heads=2, q_heads=8, head_dim=D, code_bits=bits,
                 qmax=qmax)
    p, s = build(w, 700)
    q = torch.zeros(w.batch, w.q_heads, w.head_dim, dtype=torch.bfloat16)
    got, _ = p.decode(q)
    err = max_abs(got, p.decode_ref(q))
    note(f"decode zero query D={D} bits={bits}: max-abs {err:.3e}")
    assert err <= TOL


@needs_gpu
@pytest.mark.parametrize("splits", [0, 5, 24])
def test_decode_back_to_back_on_one_workspace(splits):
    """Calls queued back to back on one workspace each see their own partials.

    The split partials are merged by the last workgroup of each (batch, KV
    head); a stale or early read would mix in the previous call's values.
    """
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=4, q_heads=16)
    p, s = build(w, 2000)
    qs = [ks.decode_query(s) for _ in range(4)]
    refs = [p.decode_ref(q) for q in qs]
    ws = p.cache.workspace(w.q_heads)
    outs = []
    note(f"decode back to back splits={splits}")
    for q in qs + qs:
        out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
        p.cache.decode_attn(q.cuda(), out, ws, num_splits=splits)
        outs.append(out)
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        assert max_abs(out.cpu().numpy(), refs[i % 4]) <= TOL, i
    assert not ws[:64].any()


@needs_gpu
def test_decode_graph_replay_matches_eager():
    """A decode call captured in a HIP graph reproduces the eager output on
    every replay, with eager calls on the same workspace in between."""
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=8)
    p, s = build(w, 1000)
    q = ks.decode_query(s).cuda()
    ws = p.cache.workspace(w.q_heads)
    eager = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    p.cache.decode_attn(q, eager, ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    note("decode graph capture")
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            p.cache.decode_attn(q, out, ws, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    other = torch.empty_like(eager)
    for r in range(3):
        out.zero_()
        p.cache.decode_attn(ks.decode_query(s).cuda(), other, ws)   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r


@needs_gpu
@pytest.mark.parametrize("splits", [0, 8, 33, 64])
def test_decode_many_calls_one_workspace(splits):
    """96 calls queued back to back on one workspace, alternating over two
    caches and four queries: every output is right, so no workgroup ever
    merges a stale or missing partial, and the arrival counters end at 0."""
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=4, q_heads=16)
    pairs = [build(w, n, seed=seed)[0] for n, seed in ((1900, 3), (2600, 4))]
    s = ks.Stream(w, seed=5)
    qs = [ks.decode_query(s) for _ in range(4)]
    refs = [[p.decode_ref(q) for q in qs] for p in pairs]
    ws = pairs[0].cache.workspace(w.q_heads)
    outs = []
    note(f"decode 96 calls splits={splits}")
    for i in range(96):
        out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
        pairs[i % 2].cache.decode_attn(qs[(i // 2) % 4].cuda(), out, ws, num_splits=splits)
        outs.append(out)
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        assert max_abs(out.cpu().numpy(), refs[i % 2][(i // 2) % 4]) <= TOL, i
    assert not ws[:64].any()
