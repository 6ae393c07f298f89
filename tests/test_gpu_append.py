"""GPU parity of kvq_append: codes, scales, tail ring and counters bit-exact.

Every case runs the library through the C ABI and the oracle on the same
seeded inputs and compares the whole device buffers with the oracle's images.
"""
import numpy as np
import pytest
import torch

import kvq_synth as ks
from harness import Pair, note

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


def run(w, sizes, capacity, check_each=True, seed=None):
    p = Pair(w, capacity)
    s = ks.Stream(w, seed)
    for i, n in enumerate(sizes):
        k, v = ks.kv_pair(s, n)
        note(f"append {w.name} step {i} n={n}")
        p.append(k, v)
        p.check_state()
        if check_each or i == len(sizes) - 1:
            p.check_buffers()
    return p


@needs_gpu
def test_tiny_prefill_then_single_tokens():
    w = ks.TINY
    run(w, [w.prefill] + [1] * w.steps, capacity=128)


@needs_gpu
@pytest.mark.parametrize("bits,qmax,D", [(8, 127, 128), (4, 7, 128), (2, 1, 128), (4, 7, 64),
                                         (2, 1, 64), (8, 127, 32), (4, 7, 32), (8, 7, 16)])
def test_grouped_flush_small(bits, qmax, D):
    w = ks.small(ks.APPEND_INT4, batch=2, kv_heads=3, head_dim=D, code_bits=bits, qmax=qmax,
                 residual=96 if D != 16 else 64, group=128 if D != 16 else 64)
    # prefill with a ragged remainder, then ragged appends crossing flushes
    run(w, [300, 16, 1, 77, 0, 130, 5, 200], capacity=1024)


@needs_gpu
@pytest.mark.parametrize("bits,qmax,D", [(4, 7, 32), (2, 1, 64), (8, 7, 16), (4, 5, 128)])
def test_overflow_only_segments_subbyte(bits, qmax, D):
    # group 0: segments start anywhere, so packed Value words are shared
    # between segments (read-modify-write of the older fields).
    w = ks.small(ks.TINY, batch=2, kv_heads=2, q_heads=2, head_dim=D, code_bits=bits, qmax=qmax,
                 residual=5, group=0, kv_dtype="bf16", outlier_channels=(1,))
    run(w, [70, 1, 3, 1, 9, 33, 2, 64, 1, 1], capacity=256)


@needs_gpu
def test_fp32_inputs_grouped():
    w = ks.small(ks.APPEND_INT8, batch=1, kv_heads=2, head_dim=64, code_bits=4, qmax=7,
                 residual=64, group=64, kv_dtype="f32")
    run(w, [200, 33, 64, 1], capacity=512)


@needs_gpu
@pytest.mark.parametrize("w", [ks.APPEND_INT8, ks.APPEND_INT4], ids=lambda w: w.name)
def test_append_workload_full_size(w):
    # 16 x 8 heads x d128: 4096 prefill then 128 appends of 16 (16 flushes).
    p = Pair(w, w.prefill + w.steps * w.step_tokens)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, w.prefill)
    note(f"append {w.name} prefill")
    p.append(k, v)
    p.check_state()
    for i in range(w.steps):
        k, v = ks.kv_pair(s, w.step_tokens)
        p.append(k, v)
        p.check_state()
    note(f"append {w.name} compare buffers")
    p.check_buffers()
    assert p.cache.state.quantized == 6016 and p.cache.state.tail == 128


@needs_gpu
def test_earlier_segments_never_rewritten():
    w = ks.small(ks.APPEND_INT4, batch=1, kv_heads=2, head_dim=128)
    p = Pair(w, 1024)
    s = ks.Stream(w)
    k, v = ks.kv_pair(s, 400)
    p.append(k, v)
    torch.cuda.synchronize()
    n0 = p.cache.state.quantized
    W = 64
    before = (p.cache.k_codes[:, :, :n0 * W].clone(), p.cache.v_codes[:, :, :n0 * W].clone(),
              p.cache.k_scale[:, :, :p.cache.state.segments].clone(), p.cache.v_scale[:, :, :n0].clone())
    for n in (100, 200, 3):
        k, v = ks.kv_pair(s, n)
        p.append(k, v)
    torch.cuda.synchronize()
    after = (p.cache.k_codes[:, :, :n0 * W], p.cache.v_codes[:, :, :n0 * W],
             p.cache.k_scale[:, :, :before[2].shape[2]], p.cache.v_scale[:, :, :n0])
    for x, y in zip(before, after):
        assert torch.equal(x, y)
    assert p.cache.state.quantized > n0


@needs_gpu
def test_zero_inputs_give_saturated_scales_and_zero_codes():
    w = ks.small(ks.APPEND_INT4, batch=1, kv_heads=1, head_dim=64, residual=64, group=64)
    p = Pair(w, 256)
    z = torch.zeros(1, 1, 200, 64, dtype=torch.bfloat16)
    p.append(z, z)
    p.check_buffers()
    torch.cuda.synchronize()
    assert torch.all(p.cache.k_scale[:, :, :p.cache.state.segments] == 65504)
    assert not p.cache.k_codes.any() and not p.cache.v_codes.any()
