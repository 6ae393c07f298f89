"""kvq_decode_attn_noalloc (no workspace, no allocation) against
kvq_decode_attn on the same caches and queries: two calls in a row, the
second on a smaller cache, each output equal to the workspace entry point's
(the same kernels and split count: bit for bit) and within the parity bar of
the oracle."""
import math

import numpy as np
import pytest
import torch

import kvq_synth as ks
import quantized_kv_cache_kvq_amd as kvq
from harness import Pair, max_abs, note

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


@needs_gpu
def test_noalloc_matches_workspace_entry_point():
    shapes = [(ks.small(ks.LLAMA3_DECODE, batch=4, kv_heads=4, q_heads=16), 3000, 0),
              (ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=8), 700, 3)]
    for i, (w, n, splits) in enumerate(shapes):
        p = Pair(w, n + 128)
        s = ks.Stream(w, seed=40 + i)
        k, v = ks.kv_pair(s, n)
        p.append(k, v)
        q = ks.decode_query(s).cuda()
        ws = p.cache.workspace(w.q_heads)
        ref_out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device="cuda")
        got = torch.full_like(ref_out, float("nan"))
        sigma = 1.0 / math.sqrt(w.head_dim)
        note(f"noalloc call {i}: batch {w.batch}, {n} tokens, splits {splits}")
        kvq.kvq_decode_attn(p.cfg, p.cache.state, p.cache.c, q, w.q_heads, sigma, splits, ref_out, ws)
        kvq.kvq_decode_attn_noalloc(p.cfg, p.cache.state, p.cache.c, q, w.q_heads, sigma, splits, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_out), i
        assert max_abs(got.cpu().numpy(), p.decode_ref(q.cpu())) <= 2e-3


@needs_gpu
def test_noalloc_rejects_partials_beyond_its_array():
    w = ks.small(ks.LLAMA3_DECODE, batch=64, kv_heads=8, q_heads=64)
    p = Pair(w, 256)
    s = ks.Stream(w, seed=9)
    k, v = ks.kv_pair(s, 200)
    p.append(k, v)
    q = ks.decode_query(s).cuda()
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    # 64 x 64 query rows x 256 splits x 132 floats is far beyond 8 MiB
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_decode_attn_noalloc(p.cfg, p.cache.state, p.cache.c, q, w.q_heads, 0.1, 256, out)
    assert e.value.status == kvq.KVQ_EWORKSPACE
