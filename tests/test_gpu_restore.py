"""GPU parity of kvq_restore against the oracle's restore, bit for bit.

restore = code / max(scale, eps) ("KV Cache Quantization Strategies", Step 4),
an IEEE fp32 division on both sides; the bf16 output is that value rounded
once to nearest even.
"""
import numpy as np
import pytest
import torch

import kvq_synth as ks
from harness import Pair, note
from oracle.cache import key_scales, segment_of_tokens, stacked_codes, value_scales
from oracle.codec import restore

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


def oracle_restore(p):
    """fp32 restored prefix [B, H, Nq, D] of keys and values from the oracle state."""
    o = p.ost
    kc, vc = stacked_codes(o, "key"), stacked_codes(o, "value")
    seg = segment_of_tokens(o)
    ks_ = key_scales(o).astype(np.float32)[:, :, seg]              # [B, H, Nq, D]
    vs_ = value_scales(o).astype(np.float32)[:, :, :, None]         # [B, H, Nq, 1]
    return restore(kc, ks_, 1e-8, np.float32), restore(vc, vs_, 1e-8, np.float32)


def run(p, dtype, pad=5):
    c = p.cache
    B, H, D = p.cfg.batch, p.cfg.kv_heads, p.cfg.head_dim
    nq = c.state.quantized
    k = torch.full((B, H, nq + pad, D), float("nan"), dtype=dtype, device="cuda")
    v = torch.full_like(k, float("nan"))
    c.restore(k, v)
    torch.cuda.synchronize()
    return k.float().cpu().numpy(), v.float().cpu().numpy()


@needs_gpu
@pytest.mark.parametrize("D,bits,qmax,group,n", [
    (128, 4, 7, 128, 1000),
    (128, 2, 1, 128, 700),
    (128, 8, 127, 128, 400),
    (64, 4, 7, 128, 600),
    (32, 8, 127, 128, 300),
    (16, 8, 127, 64, 200),
])
def test_restore_bit_exact(D, bits, qmax, group, n):
    w = ks.small(ks.LLAMA3_DECODE, batch=2, kv_heads=2, q_heads=4, head_dim=D, code_bits=bits, qmax=qmax,
                 group=group)
    p = Pair(w, n + 128)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, n)
    p.append(k, v)
    note(f"restore D={D} bits={bits} n={n}")
    nq = p.cache.state.quantized
    assert nq > 0
    ek, ev = oracle_restore(p)
    gk, gv = run(p, torch.float32)
    assert np.array_equal(gk[:, :, :nq], ek) and np.array_equal(gv[:, :, :nq], ev)
    assert np.isnan(gk[:, :, nq:]).all() and np.isnan(gv[:, :, nq:]).all()     # rows past the prefix untouched
    bk, bv = run(p, torch.bfloat16)
    rk = torch.from_numpy(ek).to(torch.bfloat16).float().numpy()
    rv = torch.from_numpy(ev).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bk[:, :, :nq], rk) and np.array_equal(bv[:, :, :nq], rv)


@needs_gpu
def test_restore_overflow_only_segments_and_empty_prefix():
    w = ks.small(ks.TINY, batch=2, kv_heads=2, q_heads=4, head_dim=64, code_bits=4, qmax=7,
                 residual=10, group=0, kv_dtype="bf16")
    p = Pair(w, 512)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, 8)              # inside the window: nothing quantized yet
    p.append(k, v)
    assert p.cache.state.quantized == 0
    gk, _ = run(p, torch.float32)
    assert np.isnan(gk).all()
    for n in (100, 1, 7, 64, 3):
        k, v = ks.kv_pair(s, n)
        p.append(k, v)
    nq = p.cache.state.quantized
    ek, ev = oracle_restore(p)
    gk, gv = run(p, torch.float32)
    assert np.array_equal(gk[:, :, :nq], ek) and np.array_equal(gv[:, :, :nq], ev)
