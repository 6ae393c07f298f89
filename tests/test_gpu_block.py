"""GPU parity of kvq_block_attn against the fp64 oracle (max-abs 2e-3).

Causal block attention: query i of the block sees every cached token and
block tokens 0..i ("KV Cache and autoregressive video generation", section
3.1).  The oracle restores the codes it produced itself, which the append
tests show are byte-identical to the device's.
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
    k, v = ks.kv_pair(s, n)          # n = 0: an empty append (a no-op) gives the empty state
    note(f"block build {w.name} n={n}")
    p.append(k, v)
    return p, s


@needs_gpu
@pytest.mark.parametrize("D,bits,qmax,g,n,tq", [
    (128, 2, 1, 4, 1000, 100),    # int2 like the video cache; ragged tiles everywhere
    (128, 4, 7, 4, 700, 64),
    (128, 8, 127, 2, 600, 33),
    (64, 2, 1, 8, 500, 70),
    (64, 4, 7, 1, 900, 130),
    (128, 4, 7, 8, 257, 17),
])
def test_block_shapes(D, bits, qmax, g, n, tq):
    w = ks.small(ks.VIDEO_BLOCK, batch=2, kv_heads=2, q_heads=2 * g, head_dim=D, code_bits=bits,
                 qmax=qmax, residual=128, group=128)
    p, s = build(w, n)
    q, kb, vb = ks.block_inputs(s, tq)
    note(f"block D={D} bits={bits} g={g} n={n} tq={tq}")
    got = p.block(q, kb, vb)
    ref = p.block_ref(q, kb, vb)
    err = max_abs(got, ref)
    note(f"block D={D} bits={bits} g={g} n={n} tq={tq}: max-abs {err:.3e}")
    assert err <= TOL


@needs_gpu
@pytest.mark.parametrize("splits", [1, 2, 3, 8])
def test_block_split_invariance(splits):
    w = ks.small(ks.VIDEO_BLOCK, batch=1, kv_heads=2, q_heads=8)
    p, s = build(w, 1500)
    q, kb, vb = ks.block_inputs(s, 40)
    ref = p.block_ref(q, kb, vb)
    note(f"block splits={splits}")
    got = p.block(q, kb, vb, num_splits=splits)
    assert max_abs(got, ref) <= TOL


@needs_gpu
@pytest.mark.parametrize("n", [0, 1, 100, 128, 129, 300])
def test_block_short_caches(n):
    """Empty cache, tail only, exactly one group, one token past a flush."""
    w = ks.small(ks.VIDEO_BLOCK, batch=1, kv_heads=2, q_heads=8, code_bits=4, qmax=7)
    p, s = build(w, n, capacity=512)
    q, kb, vb = ks.block_inputs(s, 50)
    note(f"block short cache n={n}")
    got = p.block(q, kb, vb)
    ref = p.block_ref(q, kb, vb)
    assert max_abs(got, ref) <= TOL


@needs_gpu
@pytest.mark.parametrize("D", [64, 128])
def test_block_overflow_only_segments(D):
    """Per-append segments (one Key-scale row per flush, of any length)."""
    w = ks.small(ks.TINY, batch=2, kv_heads=2, q_heads=8, head_dim=D, code_bits=4, qmax=7,
                 residual=10, group=0, kv_dtype="bf16")
    p = Pair(w, 1024)
    s = ks.Stream(w)
    for n in (100, 1, 7, 64, 3, 200, 65):
        k, v = ks.kv_pair(s, n)
        p.append(k, v)
    q, kb, vb = ks.block_inputs(s, 37)
    note(f"block overflow-only segments D={D}")
    got = p.block(q, kb, vb)
    ref = p.block_ref(q, kb, vb)
    err = max_abs(got, ref)
    note(f"block overflow-only segments D={D}: max-abs {err:.3e}")
    assert err <= TOL


@needs_gpu
@pytest.mark.parametrize("frame,n,tq,splits", [
    (4, 1000, 100, 0),       # frames straddle the cache end (N = 1000 is not a multiple of 4 * 64)
    (100, 1000, 300, 0),     # N a whole number of frames
    (64, 900, 200, 3),
    (37, 777, 150, 1),       # odd frame length, ragged tiles
    (1300, 1000, 256, 0),    # one frame spans the block: bidirectional
])
def test_block_frames(frame, n, tq, splits):
    """Frames of F positions: bidirectional inside a frame, causal across
    frames ("KV Cache and autoregressive video generation", section 6.3)."""
    w = ks.small(ks.VIDEO_BLOCK, batch=1, kv_heads=2, q_heads=8)
    p, s = build(w, n)
    q, kb, vb = ks.block_inputs(s, tq)
    note(f"block frames F={frame} n={n} tq={tq} splits={splits}")
    got = p.block(q, kb, vb, num_splits=splits, frame_tokens=frame)
    ref = p.block_ref(q, kb, vb, frame_tokens=frame)
    err = max_abs(got, ref)
    note(f"block frames F={frame}: max-abs {err:.3e}")
    assert err <= TOL


@needs_gpu
def test_block_frame_of_one_is_token_causal():
    w = ks.small(ks.VIDEO_BLOCK, batch=1, kv_heads=2, q_heads=8, code_bits=4, qmax=7)
    p, s = build(w, 700)
    q, kb, vb = ks.block_inputs(s, 90)
    assert np.array_equal(p.block(q, kb, vb), p.block(q, kb, vb, frame_tokens=1))
    with pytest.raises(Exception):
        p.block(q, kb, vb, frame_tokens=0)


@needs_gpu
def test_block_of_one_equals_decode_after_append():
    """tq = 1: the block path equals appending the token, then decoding."""
    w = ks.small(ks.VIDEO_BLOCK, batch=2, kv_heads=2, q_heads=8, code_bits=4, qmax=7)
    p, s = build(w, 900)
    q, kb, vb = ks.block_inputs(s, 1)
    note("block tq=1 vs decode")
    got_block = p.block(q, kb, vb)[:, 0]
    p.append(kb.transpose(1, 2).contiguous(), vb.transpose(1, 2).contiguous())
    got_dec, _ = p.decode(q[:, 0].contiguous())
    ref = p.decode_ref(q[:, 0].contiguous())
    assert max_abs(got_block, ref) <= TOL
    assert max_abs(got_dec, ref) <= TOL
    assert max_abs(got_block, got_dec) <= TOL


@needs_gpu
def test_block_rejects_unsupported():
    w = ks.small(ks.TINY, batch=1, kv_heads=2, q_heads=2)       # fp32 K/V, head_dim 16
    p, s = build(w, 20, capacity=64)
    q = torch.zeros(1, 4, 2, 16)
    with pytest.raises(Exception):
        p.block(q, torch.zeros(1, 4, 2, 16), torch.zeros(1, 4, 2, 16))


@needs_gpu
def test_block_video_full_size():
    """The video block at full size: 432000 int2 tokens (codes, scales and
    counters of the whole cache bit-exact against the oracle), then 1024
    queries, token-causal and in frames of 14400 positions (the block then
    lies inside one frame and is bidirectional).  The fp64 oracle computes
    64 query rows (0, 1023 and a seeded spread) for all 32 query heads; the
    kernel computes every row."""
    w = ks.VIDEO_BLOCK
    p, s = build(w, w.prefill)
    note("block video full size: buffers")
    p.check_state()
    p.check_buffers()
    q, kb, vb = ks.block_inputs(s, w.block_q)
    rng = np.random.default_rng(5)
    rest = np.setdiff1d(np.arange(1, w.block_q - 1), [511])
    rows = np.unique(np.concatenate(([0, 511, w.block_q - 1], rng.choice(rest, 61, replace=False))))
    assert rows.size == 64
    for frame in (1, 14400):
        note(f"block video full size frames={frame}")
        got = p.block(q, kb, vb, frame_tokens=frame)
        assert np.isfinite(got).all()
        ref = p.block_ref(q, kb, vb, rows=rows, frame_tokens=frame)
        err = max_abs(got[:, rows], ref[:, rows])
        note(f"block video full size frames={frame}: max-abs {err:.3e} over {rows.size} rows x {w.q_heads} heads")
        assert err <= TOL


@needs_gpu
def test_block_fp8_low_part_scales():
    """The powers of two of the fp8 low product: one Key segment eight times
    larger than the rest (so the smallest Key scale, and with it the
    workgroup's power of two, comes from one segment of its run) and query
    rows of very different size inside one wave (every other position a
    64th of the others, which sets the wave's query power of two).  Same
    oracle bound as every block test."""
    w = ks.small(ks.VIDEO_BLOCK, batch=1, kv_heads=2, q_heads=8)
    p = Pair(w, 1200)
    s = ks.Stream(w, 77)
    k, v = ks.kv_pair(s, 1100)
    k[:, :, 256:384] *= 8                        # one 128-token segment (the third)
    p.append(k, v)
    q, kb, vb = ks.block_inputs(s, 96)
    q[:, 1::2] /= 64                             # rows of one wave differ by 2^6
    note("block fp8 low-part scales")
    got = p.block(q, kb, vb, num_splits=3)
    err = max_abs(got, p.block_ref(q, kb, vb))
    note(f"block fp8 low-part scales: max-abs {err:.3e}")
    assert err <= TOL
