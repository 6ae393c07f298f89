"""Pins for the oracle's same-axis mode (Keys and Values both per token, one
scale per run of 64 channels: "KV Cache Quantization Strategies", Step 2
table, third row, in the setting of that page's section 5.1).

Fixed by: a token worked by hand (one outlier channel coarsens only its own
run), history independence (a per-token scale cannot depend on how the
tokens were appended, unlike KIVI's per-segment Key scale), and inputs on
power-of-two grids that restore exactly, so the oracle's decode attention
over the quantized cache must equal the plain definition over the raw rows
(a scale taken from the wrong run or token breaks the equality).
"""
import numpy as np
import pytest

from oracle import attention
from oracle.cache import KVQuantizationStrategies, key_scales, stacked_codes, value_scales


def _oracle(**kw):
    return KVQuantizationStrategies(qmax=kw.pop("qmax", 7), eps=1e-8, scale_storage="fp16",
                                    axis_group=64, **kw)


def test_hand_worked_token():
    """One 128-channel token, residual 1, so the first of two tokens is
    quantized.  Run 0: every value 1.0 except channel 3 = 10.0; run 1: every
    value 0.5 except channel 100 = -0.25.

    Run 0: scale = 7 / 10 = 0.7, stored as fp16 0.7001953125; codes
    round(1.0 * 0.700195) = 1 and round(10 * 0.700195) = round(7.00195) = 7.
    Run 1: scale = 7 / 0.5 = 14 (exact in fp16); codes 0.5 * 14 = 7 and
    -0.25 * 14 = -3.5, which rounds half to even to -4.
    Keys and Values quantize the same way."""
    x = np.ones((1, 1, 2, 128), np.float32)
    x[..., 3] = 10.0
    x[..., 64:] = 0.5
    x[..., 100] = -0.25
    st = _oracle().append_and_partition(None, x, x.copy(), 1)
    assert st["quantized_tokens"] == 1
    for which, scales in (("key", key_scales(st)), ("value", value_scales(st))):
        codes = stacked_codes(st, which)[0, 0, 0].astype(int)
        expect = np.r_[np.ones(64, int), np.full(64, 7)]
        expect[3] = 7
        expect[100] = -4
        assert np.array_equal(codes, expect), which
        assert scales.shape == (1, 1, 1, 2)
        assert scales[0, 0, 0, 0] == np.float16(0.7001953125) and float(scales[0, 0, 0, 0]) == 0.7001953125
        assert float(scales[0, 0, 0, 1]) == 14.0


def test_kivi_mode_differs_on_the_same_token():
    """The contrast the mode exists for: in KIVI mode the two tokens' Keys
    share a per-channel range, so the same input gives other Key codes."""
    x = np.ones((1, 1, 3, 128), np.float32)
    x[..., 0, 3] = 10.0
    x[..., 1, :] = 0.1
    kivi = KVQuantizationStrategies(qmax=7, eps=1e-8, scale_storage="fp16")
    a = stacked_codes(kivi.append_and_partition(None, x, x, 1), "key")
    b = stacked_codes(_oracle().append_and_partition(None, x, x, 1), "key")
    assert a.shape == b.shape == (1, 1, 2, 128)
    assert not np.array_equal(a, b)
    # same-axis: token 1 (all 0.1) gets the full code range in both runs
    assert np.all(b[0, 0, 1] == 7)


@pytest.mark.parametrize("group", [0, 64])
def test_codes_do_not_depend_on_how_tokens_were_appended(group):
    """Ragged appends and one append of the same rows flush the same tokens
    (up to the last whole group) and give identical codes and scales."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((2, 3, 300, 128)).astype(np.float32)
    v = rng.standard_normal((2, 3, 300, 128)).astype(np.float32)
    k[..., 7] *= 10
    o = _oracle(group=group)
    st = None
    edges = [0, 1, 17, 64, 65, 140, 203, 300]
    for lo, hi in zip(edges[:-1], edges[1:]):
        st = o.append_and_partition(st, k[:, :, lo:hi], v[:, :, lo:hi], 16)
    one = o.append_and_partition(None, k, v, 16)
    n = st["quantized_tokens"]
    assert n == one["quantized_tokens"] and n > 200
    for which in ("key", "value"):
        assert np.array_equal(stacked_codes(st, which), stacked_codes(one, which))
    assert np.array_equal(key_scales(st), key_scales(one))
    assert np.array_equal(value_scales(st), value_scales(one))
    assert key_scales(st).shape == (2, 3, n, 2)


def _grid_rows(rng, shape, qmax):
    """Rows whose every run of 64 channels is exactly representable: codes in
    [-qmax, qmax] with one element at +-qmax, divided by a power-of-two scale
    drawn per (token, run), so quantization and restore are exact."""
    B, H, T, D = shape
    codes = rng.integers(-qmax, qmax + 1, size=(B, H, T, D // 64, 64))
    codes[..., 0] = np.where(rng.random((B, H, T, D // 64)) < 0.5, qmax, -qmax)
    scale = 2.0 ** rng.integers(-3, 4, size=(B, H, T, D // 64, 1))
    return (codes / scale).reshape(B, H, T, D).astype(np.float32)


def test_decode_attention_over_exact_grid_equals_the_definition():
    rng = np.random.default_rng(9)
    B, H, D, g = 2, 2, 128, 4
    k = _grid_rows(rng, (B, H, 200, D), 7)
    v = _grid_rows(rng, (B, H, 200, D), 7)
    st = _oracle(group=64).append_and_partition(None, k, v, 40)
    assert st["quantized_tokens"] == 128
    q = rng.standard_normal((B, H * g, D))
    got = attention.decode_attention(st, q, 0.125)
    for b in range(B):
        for h in range(H):
            ref = attention.attention_rows(q[b, h * g:(h + 1) * g], k[b, h], v[b, h], 0.125)
            assert np.allclose(got[b, h * g:(h + 1) * g], ref, rtol=0, atol=1e-12)
    # and the restored prefix is the input itself
    k_hat, v_hat = attention.restored_cache(st, 1, 0)
    assert np.array_equal(k_hat, k[1, 0].astype(np.float64))
    assert np.array_equal(v_hat, v[1, 0].astype(np.float64))
