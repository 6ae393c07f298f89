"""GPU parity of the paged cache: per-sequence lengths and a block table.

Every sequence of a paged cache must behave exactly like a cache of its own
(the same codes, scales, window and counters as the oracle run on that
sequence alone), with its 64-token tiles in the pages its row of the block
table names ("KV Cache and autoregressive video generation", section 05: a
block table maps logical blocks to physical ones; "KV Cache quantization and
compression", section 07: the low-bit data and its metadata are paged
together).  Covered: kvq_paged_append (ragged and uneven counts, flushes per
sequence), kvq_paged_decode_attn (shapes, split choices, the benchmarked
size), kvq_paged_decode_step (against the oracle and against the two calls)
kvq_paged_block_attn (frames, splits, an empty prefix) and kvq_paged_restore
(bit-exact); error paths leave every state unchanged.
"""
import math

import numpy as np
import pytest
import torch

import kvq_synth as ks
import quantized_kv_cache_kvq_amd as kvq
from harness import f32, max_abs, note
from oracle import attention as oatt
from oracle import layout as olay
from oracle.cache import KVQuantizationStrategies, key_scales, stacked_codes, value_scales

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

TOL = 2e-3


class PagedPair:
    """A paged device cache and one oracle state per sequence."""

    def __init__(self, w, stride, spare=7, seed=0):
        self.w = w
        self.stride = stride
        self.cfg = kvq.make_config(batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim,
                                   capacity=stride * 64, code_bits=w.code_bits, qmax=w.qmax,
                                   residual=w.residual, group=w.group,
                                   kv_dtype=kvq.KVQ_BF16 if w.kv_dtype == "bf16" else kvq.KVQ_F32)
        self.n_pages = w.batch * stride + spare
        perm = np.random.default_rng(seed).permutation(self.n_pages)[:w.batch * stride]
        self.table_np = perm.reshape(w.batch, stride).astype(np.int32)     # shuffled pages
        self.cache = kvq.PagedKVCache(self.cfg, self.n_pages, torch.from_numpy(self.table_np).cuda())
        self.oracle = KVQuantizationStrategies(qmax=w.qmax, eps=1e-8, scale_storage="fp16", group=w.group)
        self.ost = [None] * w.batch

    def append(self, k, v, lens):
        """k, v: CPU [B, H, max_n, D]; sequence b takes its first lens[b] rows."""
        self.cache.append(k.cuda(), v.cuda(), lens)
        for b, n in enumerate(lens):
            self.ost[b] = self.oracle.append_and_partition(
                self.ost[b], f32(k[b:b + 1, :, :n]), f32(v[b:b + 1, :, :n]), self.w.residual)

    def decode(self, q, num_splits=0):
        hq = q.shape[1]
        ws = self.cache.workspace(hq)
        out = torch.full((q.shape[0], hq, self.w.head_dim), float("nan"), device="cuda")
        self.cache.decode_attn(q.cuda(), out, ws, num_splits=num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def step(self, k, v, lens, q, num_splits=0):
        """One kvq_paged_decode_step; the oracle states advance with the same append."""
        hq = q.shape[1]
        ws = self.cache.workspace(hq)
        out = torch.full((q.shape[0], hq, self.w.head_dim), float("nan"), device="cuda")
        self.cache.decode_step(k.cuda(), v.cuda(), lens, q.cuda(), out, ws, num_splits=num_splits)
        torch.cuda.synchronize()
        for b, n in enumerate(lens):
            self.ost[b] = self.oracle.append_and_partition(
                self.ost[b], f32(k[b:b + 1, :, :n]), f32(v[b:b + 1, :, :n]), self.w.residual)
        return out.cpu().numpy()

    def decode_ref(self, q):
        sigma = 1.0 / math.sqrt(self.w.head_dim)
        return np.concatenate([oatt.decode_attention(o, f32(q[b:b + 1]), sigma) for b, o in enumerate(self.ost)])

    def check(self):
        torch.cuda.synchronize()
        w, H, D = self.w, self.w.kv_heads, self.w.head_dim
        W = D * w.code_bits // 8
        head = 128 * W + 128 + 2 * D
        pool = self.cache.pool.cpu().numpy().reshape(self.n_pages, H, head)
        k_tail = f32(self.cache.k_tail)
        v_tail = f32(self.cache.v_tail)
        for b, o in enumerate(self.ost):
            st = self.cache.states[b]
            assert (st.quantized, st.tail, st.total, st.segments) == (
                o["quantized_tokens"], o["key_residual"].shape[-2], o["total_tokens"], len(o["key_q_segments"]))
            nq, nt = st.quantized, st.tail
            cap = self.stride * 64
            ek = olay.pack_cache(stacked_codes(o, "key"), w.code_bits, cap, "key")[0]     # [H, stream]
            ev = olay.pack_cache(stacked_codes(o, "value"), w.code_bits, cap, "value")[0]
            eks = key_scales(o).astype(np.float16).view(np.uint16)[0]                     # [H, nseg, D]
            evs = value_scales(o).astype(np.float16).view(np.uint16)[0]                   # [H, nq]
            for j in range((nq + 63) // 64):
                page = pool[self.table_np[b, j]]                                          # [H, head]
                assert np.array_equal(page[:, :64 * W], ek[:, j * 64 * W:(j + 1) * 64 * W]), (b, j, "key codes")
                assert np.array_equal(page[:, 64 * W:128 * W], ev[:, j * 64 * W:(j + 1) * 64 * W]), (b, j, "values")
                n = min(64, nq - 64 * j)
                vs = page[:, 128 * W:128 * W + 128].copy().view(np.uint16)[:, :n]
                assert np.array_equal(vs, evs[:, 64 * j:64 * j + n]), (b, j, "value scales")
                ksr = page[:, 128 * W + 128:].copy().view(np.uint16)
                assert np.array_equal(ksr, eks[:, (64 * j) // w.group]), (b, j, "key scales")
            slots = olay.ring_positions(nq, nt, self.cache.ring)
            assert np.array_equal(k_tail[b][:, slots], o["key_residual"][0])
            assert np.array_equal(v_tail[b][:, slots], o["value_residual"][0])


@needs_gpu
@pytest.mark.parametrize("bits,qmax", [(4, 7), (2, 1), (8, 127)])
def test_paged_ragged_prefill_decode_steps(bits, qmax):
    w = ks.small(ks.LLAMA3_DECODE, batch=3, kv_heads=2, q_heads=8, code_bits=bits, qmax=qmax)
    p = PagedPair(w, stride=24, seed=bits)
    s = ks.Stream(w)
    lens = [300, 1000, 129]
    k, v = ks.kv_pair(s, max(lens))
    note(f"paged bits={bits} prefill {lens}")
    p.append(k, v, lens)
    p.check()
    worst = 0.0
    nq0 = [p.cache.states[b].quantized for b in range(3)]
    for step in range(30):                 # sequence 1 reaches residual + group tokens at step 24
        q = ks.decode_query(s)
        got = p.decode(q)
        worst = max(worst, max_abs(got, p.decode_ref(q)))
        k1, v1 = ks.kv_pair(s, 1)
        p.append(k1, v1, [1, 1, 1])
    p.check()
    assert p.cache.states[1].quantized > nq0[1]    # a flush inside the decode steps
    note(f"paged bits={bits}: max-abs {worst:.3e}")
    assert worst <= TOL


@needs_gpu
def test_paged_uneven_appends_flush_per_sequence():
    """Sequences append different counts (0 included); each flushes on its own."""
    w = ks.small(ks.LLAMA3_DECODE, batch=4, kv_heads=2, q_heads=4, head_dim=64, code_bits=4, qmax=7)
    p = PagedPair(w, stride=20, seed=9)
    s = ks.Stream(w)
    plan = [[200, 0, 130, 1], [5, 90, 0, 1], [128, 128, 256, 0], [1, 1, 1, 300], [0, 60, 3, 17]]
    for lens in plan:
        k, v = ks.kv_pair(s, max(lens))
        note(f"paged uneven {lens}")
        p.append(k, v, lens)
    p.check()
    for splits in (0, 1, 5):
        q = ks.decode_query(s)
        assert max_abs(p.decode(q, num_splits=splits), p.decode_ref(q)) <= TOL


@needs_gpu
def test_paged_rejects_bad_calls():
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=8)
    p = PagedPair(w, stride=4)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, 300)
    big_k, big_v = ks.kv_pair(s, 600)
    with pytest.raises(kvq.KVQError):          # sequence 0 would quantize 512 tokens into 4 pages of 64
        p.cache.append(big_k.cuda(), big_v.cuda(), [600, 10])
    assert all(p.cache.states[b].total == 0 for b in range(2))
    with pytest.raises(kvq.KVQError):          # fp32 rows for a bf16 cache
        p.cache.append(k.float().cuda(), v.float().cuda(), [300, 10])
    with pytest.raises(kvq.KVQError):          # a count beyond the rows given
        p.cache.append(k.cuda(), v.cuda(), [301, 10])
    with pytest.raises(kvq.KVQError):          # more rows than max(n_new): the row stride would be wrong
        p.cache.append(k.cuda(), v.cuda(), [200, 10])
    assert all(p.cache.states[b].total == 0 for b in range(2))
    p.append(k, v, [300, 10])
    q = ks.decode_query(s).cuda()
    out = torch.empty(2, 8, w.head_dim, device="cuda")
    ws = p.cache.workspace(8)
    with pytest.raises(kvq.KVQError):          # q_heads not a multiple of kv_heads
        kvq.kvq_paged_decode_attn(p.cfg, p.cache.states, p.cache.c, q, 7, 0.1, 0, out, ws)
    with pytest.raises(kvq.KVQError):          # workspace too small
        kvq.kvq_paged_decode_attn(p.cfg, p.cache.states, p.cache.c, q, 8, 0.1, 0, out, ws[:8])
    p.check()


@needs_gpu
@pytest.mark.parametrize("D,bits,qmax,gqa,group,kv_dtype", [
    (64, 4, 7, 2, 64, "f32"),       # fp32 windows: the vector-ALU paged kernel
    (64, 2, 1, 8, 128, "bf16"),     # int2, eight query heads per KV head (matrix-core kernel)
    (32, 8, 127, 4, 64, "bf16"),    # head_dim 32 int8 (vector-ALU kernel)
])
def test_paged_other_shapes(D, bits, qmax, gqa, group, kv_dtype):
    w = ks.small(ks.LLAMA3_DECODE, batch=3, kv_heads=2, q_heads=2 * gqa, head_dim=D, code_bits=bits,
                 qmax=qmax, group=group, kv_dtype=kv_dtype)
    p = PagedPair(w, stride=12, seed=D + bits)
    s = ks.Stream(w)
    lens = [500, 70, 333]
    k, v = ks.kv_pair(s, max(lens))
    note(f"paged D={D} bits={bits} gqa={gqa} {kv_dtype}")
    p.append(k, v, lens)
    for step in range(3):
        q = ks.decode_query(s)
        assert max_abs(p.decode(q), p.decode_ref(q)) <= TOL
        k1, v1 = ks.kv_pair(s, 5)
        p.append(k1, v1, [5, 0, 3])
    p.check()


@needs_gpu
def test_paged_long_sequence_one_split():
    """One split over more than 64 tiles per wave takes the vector-ALU kernel
    (the matrix-core kernel keeps a wave's page numbers in its 64 lanes); the
    automatic split count takes the matrix-core kernel.  Both match the oracle."""
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=1, q_heads=4, head_dim=64)
    p = PagedPair(w, stride=300, seed=5)
    s = ks.Stream(w)
    lens = [17000, 2000]
    k, v = ks.kv_pair(s, max(lens))
    note("paged long sequence, one split")
    p.append(k, v, lens)
    q = ks.decode_query(s)
    ref = p.decode_ref(q)
    for splits in (1, 0, 2, 40):
        assert max_abs(p.decode(q, num_splits=splits), ref) <= TOL, splits
    p.check()


@needs_gpu
@pytest.mark.parametrize("bits,qmax,num_splits", [(4, 7, 0), (2, 1, 0), (4, 7, 3)])
def test_paged_decode_step(bits, qmax, num_splits):
    """kvq_paged_decode_step against the oracle and against kvq_paged_append +
    kvq_paged_decode_attn on a second cache with another page shuffle: mixed
    per-sequence counts (zeros included), steps that flush (two calls inside),
    an all-zero step."""
    w = ks.small(ks.LLAMA3_DECODE, batch=4, kv_heads=2, q_heads=8, code_bits=bits, qmax=qmax)
    fused = PagedPair(w, stride=24, seed=11)
    split = PagedPair(w, stride=24, seed=12)
    s = ks.Stream(w)
    lens = [300, 1000, 129, 200]
    k, v = ks.kv_pair(s, max(lens))
    fused.append(k, v, lens)
    split.append(k, v, lens)
    plan = [[1, 1, 1, 1], [0, 2, 1, 3], [16, 1, 0, 5], [1, 0, 0, 0], [0, 0, 0, 0], [3, 3, 3, 3]]
    worst = worst_pair = 0.0
    one_pass = flush_steps = 0
    for i in range(36):
        ns = plan[i % len(plan)]
        nxt = [kvq.kvq_plan_append(fused.cfg, fused.cache.states[b], ns[b]) for b in range(4)]
        if any(x.flushed_last for x in nxt):
            flush_steps += 1
        elif max(ns) > 0:
            one_pass += 1
        k1, v1 = ks.kv_pair(s, max(ns))
        q = ks.decode_query(s)
        note(f"paged step {i} bits={bits} n={ns}")
        got = fused.step(k1, v1, ns, q, num_splits=num_splits)
        split.append(k1, v1, ns)
        ref2 = split.decode(q, num_splits=num_splits)
        worst = max(worst, max_abs(got, fused.decode_ref(q)))
        worst_pair = max(worst_pair, max_abs(got, ref2))
    fused.check()
    split.check()
    note(f"paged step bits={bits}: max-abs {worst:.3e}, vs two calls {worst_pair:.3e}, "
         f"{one_pass} one-pass steps, {flush_steps} flush steps")
    assert worst <= TOL and worst_pair <= 1e-4
    assert one_pass >= 20 and flush_steps >= 1


@needs_gpu
def test_paged_decode_step_errors_leave_states_unchanged():
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=8)
    p = PagedPair(w, stride=8)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, 200)
    p.append(k, v, [200, 150])
    before = [(x.quantized, x.tail, x.total) for x in p.cache.states]
    k1, v1 = ks.kv_pair(s, 1)
    q = ks.decode_query(s).cuda()
    out = torch.empty(2, 8, w.head_dim, device="cuda")
    ws = p.cache.workspace(8)
    with pytest.raises(kvq.KVQError):          # q_heads not a multiple of kv_heads
        kvq.kvq_paged_decode_step(p.cfg, p.cache.states, p.cache.c, k1.cuda(), v1.cuda(), [1, 1], q, 7, 0.1, 0,
                                  out, ws)
    with pytest.raises(kvq.KVQError):          # workspace too small
        kvq.kvq_paged_decode_step(p.cfg, p.cache.states, p.cache.c, k1.cuda(), v1.cuda(), [1, 1], q, 8, 0.1, 0,
                                  out, ws[:8])
    big_k, big_v = ks.kv_pair(s, 600)
    with pytest.raises(kvq.KVQError):          # capacity: sequence 0 would quantize 640 tokens into 8 pages of 64
        p.cache.decode_step(big_k.cuda(), big_v.cuda(), [600, 1], q, out, ws)
    stage_k, stage_v = ks.kv_pair(s, 16)
    with pytest.raises(kvq.KVQError):          # a 16-row staging buffer for one token each
        p.cache.decode_step(stage_k.cuda(), stage_v.cuda(), [1, 1], q, out, ws)
    assert [(x.quantized, x.tail, x.total) for x in p.cache.states] == before
    p.check()


@needs_gpu
@pytest.mark.parametrize("bits,qmax,frame,num_splits", [(4, 7, 1, 0), (2, 1, 16, 0), (4, 7, 1, 4), (8, 127, 7, 2)])
def test_paged_block_attn(bits, qmax, frame, num_splits):
    """Block attention over paged caches: each sequence's block of tq queries
    sits after its own cached tokens; compared with the oracle run on each
    sequence alone (a sequence with an empty prefix included)."""
    w = ks.small(ks.LLAMA3_DECODE, batch=3, kv_heads=2, q_heads=8, code_bits=bits, qmax=qmax)
    p = PagedPair(w, stride=24, seed=21 + bits)
    s = ks.Stream(w)
    lens = [700, 90, 1300]
    k, v = ks.kv_pair(s, max(lens))
    p.append(k, v, lens)
    tq = 100
    q, kb, vb = ks.block_inputs(s, tq)
    ws = p.cache.workspace(w.q_heads, tq)
    out = torch.full((w.batch, tq, w.q_heads, w.head_dim), float("nan"), device="cuda")
    note(f"paged block bits={bits} F={frame} splits={num_splits}")
    p.cache.block_attn(q.cuda(), kb.cuda(), vb.cuda(), out, ws, num_splits=num_splits, frame_tokens=frame)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sigma = 1.0 / math.sqrt(w.head_dim)
    worst = 0.0
    for b, o in enumerate(p.ost):
        ref = oatt.block_attention(o, f32(q[b:b + 1]), f32(kb[b:b + 1]), f32(vb[b:b + 1]), sigma,
                                   frame_tokens=frame)
        worst = max(worst, max_abs(got[b:b + 1], ref))
    note(f"paged block bits={bits}: max-abs {worst:.3e}")
    assert worst <= TOL
    p.check()


@needs_gpu
def test_paged_decode_llama3_full_size_ragged():
    """The paged workload the benchmark times: Llama-3-8B shape (batch 8, 32 / 8
    heads, head_dim 128, int4), lengths 494 .. 7845 from the benchmark's seeded
    draw, a shuffled page table, the automatic split choice; every output
    against the oracle, then one decode step (one token per sequence)."""
    w = ks.LLAMA3_DECODE
    lens = [int(x) for x in np.random.default_rng(4096).integers(256, 7937, size=w.batch)]
    p = PagedPair(w, stride=max(lens) // 64 + 4, seed=4096)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, max(lens))
    note(f"paged full size {lens}")
    p.append(k, v, lens)
    del k, v
    q = ks.decode_query(s)
    err = max_abs(p.decode(q), p.decode_ref(q))
    k1, v1 = ks.kv_pair(s, 1)
    q1 = ks.decode_query(s)
    err1 = max_abs(p.step(k1, v1, [1] * w.batch, q1), p.decode_ref(q1))
    note(f"paged full size: max-abs {err:.3e}, step {err1:.3e}")
    assert err <= TOL and err1 <= TOL
    p.check()


@needs_gpu
def test_paged_maximum_batch_of_64_sequences():
    """64 sequences (the most a paged call takes: every per-sequence array of
    the kernel arguments full), ragged lengths including a one-token sequence:
    append, decode, one fused step and block attention against the oracle."""
    w = ks.small(ks.LLAMA3_DECODE, batch=64, kv_heads=1, q_heads=4, head_dim=64)
    p = PagedPair(w, stride=6, seed=64)
    s = ks.Stream(w)
    lens = [int(x) for x in np.random.default_rng(64).integers(1, 330, size=64)]
    lens[0], lens[1] = 1, 329
    k, v = ks.kv_pair(s, max(lens))
    note("paged batch 64")
    p.append(k, v, lens)
    q = ks.decode_query(s)
    assert max_abs(p.decode(q), p.decode_ref(q)) <= TOL
    k1, v1 = ks.kv_pair(s, 2)
    q1 = ks.decode_query(s)
    assert max_abs(p.step(k1, v1, [2] * 64, q1), p.decode_ref(q1)) <= TOL
    tq = 20
    qb, kb, vb = ks.block_inputs(s, tq)
    ws = p.cache.workspace(w.q_heads, tq)
    out = torch.full((64, tq, w.q_heads, w.head_dim), float("nan"), device="cuda")
    p.cache.block_attn(qb.cuda(), kb.cuda(), vb.cuda(), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sigma = 1.0 / math.sqrt(w.head_dim)
    for b in (0, 1, 17, 63):
        ref = oatt.block_attention(p.ost[b], f32(qb[b:b + 1]), f32(kb[b:b + 1]), f32(vb[b:b + 1]), sigma)
        assert max_abs(got[b:b + 1], ref) <= TOL, b
    p.check()


@needs_gpu
def test_paged_append_all_64_sequences_flush_in_one_call():
    """One kvq_paged_append in which every one of 64 sequences flushes (one
    or two 128-token groups, from different starting tails): all of them go
    through a single flush launch, and every page, window and counter
    matches the oracle run on that sequence alone."""
    w = ks.small(ks.LLAMA3_DECODE, batch=64, kv_heads=2, q_heads=4, head_dim=64)
    p = PagedPair(w, stride=10, seed=640)
    s = ks.Stream(w)
    first = [100 + b for b in range(64)]                  # 100 .. 163 tokens: no flush yet
    k, v = ks.kv_pair(s, max(first))
    p.append(k, v, first)
    assert all(p.cache.states[b].quantized == 0 for b in range(64))
    second = [160 + (b % 5) * 40 for b in range(64)]     # every tail passes residual + group
    nxt = [kvq.kvq_plan_append(p.cfg, p.cache.states[b], second[b]) for b in range(64)]
    assert all(x.flushed_last > 0 for x in nxt) and {x.flushed_last for x in nxt} == {128, 256}
    k, v = ks.kv_pair(s, max(second))
    note("paged append: 64 sequences flushing together")
    p.append(k, v, second)
    p.check()
    q = ks.decode_query(s)
    assert max_abs(p.decode(q), p.decode_ref(q)) <= TOL


@needs_gpu
def test_paged_decode_step_fp32_takes_the_two_calls():
    """fp32 windows: every step runs kvq_paged_append then kvq_paged_decode_attn
    inside the one call; outputs and states still match the oracle."""
    w = ks.small(ks.LLAMA3_DECODE, batch=3, kv_heads=2, q_heads=4, head_dim=64, group=64, kv_dtype="f32")
    p = PagedPair(w, stride=12, seed=32)
    s = ks.Stream(w)
    lens = [150, 400, 70]
    k, v = ks.kv_pair(s, max(lens))
    p.append(k, v, lens)
    for ns in ([1, 1, 1], [0, 3, 1], [2, 0, 0], [70, 1, 1]):
        k1, v1 = ks.kv_pair(s, max(ns))
        q = ks.decode_query(s)
        note(f"paged fp32 step n={ns}")
        assert max_abs(p.step(k1, v1, ns, q), p.decode_ref(q)) <= TOL
    p.check()


@needs_gpu
@pytest.mark.parametrize("bits,qmax,dtype", [(4, 7, torch.float32), (2, 1, torch.bfloat16), (8, 127, torch.float32)])
def test_paged_restore_bit_exact(bits, qmax, dtype):
    """kvq_paged_restore: each sequence's prefix equals the oracle's restore
    (fp32 division, or that rounded once to bf16); rows past a sequence's
    prefix are not written (an empty prefix included)."""
    from oracle.cache import segment_of_tokens
    from oracle.codec import restore
    w = ks.small(ks.LLAMA3_DECODE, batch=3, kv_heads=2, q_heads=4, code_bits=bits, qmax=qmax)
    p = PagedPair(w, stride=16, seed=7 + bits)
    s = ks.Stream(w)
    lens = [900, 100, 530]
    k, v = ks.kv_pair(s, max(lens))
    p.append(k, v, lens)
    nq = [p.cache.states[b].quantized for b in range(3)]
    ld = max(nq) + 3
    ko = torch.full((3, w.kv_heads, ld, w.head_dim), float("nan"), dtype=dtype, device="cuda")
    vo = torch.full_like(ko, float("nan"))
    note(f"paged restore bits={bits} {dtype} nq={nq}")
    p.cache.restore(ko, vo)
    torch.cuda.synchronize()
    ko, vo = ko.float().cpu().numpy(), vo.float().cpu().numpy()
    for b, o in enumerate(p.ost):
        n = nq[b]
        assert np.isnan(ko[b, :, n:]).all() and np.isnan(vo[b, :, n:]).all(), b
        if n == 0:
            continue
        seg = segment_of_tokens(o)
        ek = restore(stacked_codes(o, "key"), key_scales(o).astype(np.float32)[:, :, seg], 1e-8, np.float32)[0]
        ev = restore(stacked_codes(o, "value"), value_scales(o).astype(np.float32)[:, :, :, None], 1e-8,
                     np.float32)[0]
        if dtype == torch.bfloat16:
            ek = torch.from_numpy(ek).to(torch.bfloat16).float().numpy()
            ev = torch.from_numpy(ev).to(torch.bfloat16).float().numpy()
        assert np.array_equal(ko[b, :, :n], ek) and np.array_equal(vo[b, :, :n], ev), b
