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


def _tie_rows(qmax, n_pairs, seed):
    """(x, s, a) triples: x's float32 product with the fp16 scale s lands on a
    half-integer that its exact product misses, and a range a whose stored
    fp16 scale is s (so a row or column [a, x] quantizes x with s)."""
    from fractions import Fraction

    from exact import f32_tie_pairs, fr, nearest_f32
    out = []
    for x_t, sc in f32_tie_pairs(4 * n_pairs, qmax, seed=seed, scale_range=(2.0, 60.0)):
        a = nearest_f32(Fraction(qmax) / fr(sc))
        if np.float16(np.float32(qmax) / a) == sc and abs(x_t) <= a:
            out.append((x_t, sc, a))
        if len(out) == n_pairs:
            return out
    raise AssertionError("not enough tie pairs")


@needs_gpu
@pytest.mark.parametrize("bits,qmax,group", [(8, 7, 0), (4, 7, 64), (8, 127, 64)])
def test_fp32_product_ties_bit_exact(bits, qmax, group):
    """fp32 Keys and Values built so that the float32 product x * s of many
    elements lands exactly on a half-integer while the exact product does
    not, plus the round-half-even vector [7, 2.5, -2.5, 0.5, 1.5, -0.5, 3.5]
    (scale 1) along both axes: the codes and scales the library writes equal
    the oracle's bit for bit, and the tie elements' codes are the half-even
    rounding of the float32 product (computed here by exact arithmetic)."""
    from exact import fr, nearest_f32, round_half_even
    D, H, n = (16 if bits == 8 else 32), 2, 64
    w = ks.small(ks.TINY, batch=1, kv_heads=H, q_heads=H, head_dim=D, code_bits=bits, qmax=qmax,
                 residual=8, group=group, kv_dtype="f32")
    k = np.zeros((1, H, n + w.residual, D), np.float32)
    v = np.zeros_like(k)
    trip = _tie_rows(qmax, H * D + H * n, seed=bits * 1000 + qmax)
    expect_k, expect_v = {}, {}
    it = iter(trip)
    for h in range(H):                       # Keys: channel c holds [a, x] at tokens 2c, 2c + 1
        for c in range(D - 1):
            x_t, sc, a = next(it)
            k[0, h, 2 * c, c], k[0, h, 2 * c + 1, c] = a, x_t
            expect_k[(h, 2 * c + 1, c)] = round_half_even(fr(nearest_f32(fr(x_t) * fr(sc))))
        if qmax >= 7:                        # the tie vector down the last channel
            k[0, h, 40:47, D - 1] = [7, 2.5, -2.5, 0.5, 1.5, -0.5, 3.5]
    for h in range(H):                       # Values: token t holds [a, x, 0, ...]
        for t in range(n):
            x_t, sc, a = next(it)
            v[0, h, t, 0], v[0, h, t, 1] = a, x_t
            expect_v[(h, t, 1)] = round_half_even(fr(nearest_f32(fr(x_t) * fr(sc))))
        if qmax >= 7:
            v[0, h, n - 1, :7] = [7, 2.5, -2.5, 0.5, 1.5, -0.5, 3.5]
            v[0, h, n - 1, 7:] = 0.0
            expect_v.pop((h, n - 1, 1), None)
    p = Pair(w, 256)
    note(f"fp32 ties bits={bits} qmax={qmax} group={group}")
    p.append(torch.from_numpy(k), torch.from_numpy(v))
    p.check_state()
    p.check_buffers()                         # device bytes == oracle images
    from oracle.cache import stacked_codes
    kc, vc = stacked_codes(p.ost, "key")[0], stacked_codes(p.ost, "value")[0]
    for (h, t, c), want in expect_k.items():
        assert int(kc[h, t, c]) == max(-qmax, min(qmax, want)), ("key", h, t, c)
    for (h, t, c), want in expect_v.items():
        assert int(vc[h, t, c]) == max(-qmax, min(qmax, want)), ("value", h, t, c)
    if qmax == 7:
        assert kc[0, 40:47, D - 1].tolist() == [7, 2, -2, 0, 2, 0, 4]
        assert vc[0, n - 1, :7].tolist() == [7, 2, -2, 0, 2, 0, 4]
