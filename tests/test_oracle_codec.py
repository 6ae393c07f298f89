"""Pins for the oracle codec (quantize / restore / scale storage).

Every check here is fixed by something other than the oracle itself: the
worked grid examples printed in "KV Cache quantization and compression"
section 03, the scale-shape and zero-range contracts of "KV Cache
Quantization Strategies" Step 4 tests, the definition of round-half-to-even,
or closed-form bounds of a uniform quantizer.
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import example, given, settings, strategies as st
from hypothesis.extra import numpy as hnp

from exact import f32_tie_pairs, fr, nearest_f32, round_half_even
from oracle import codec


def product_slack(qmax):
    """Bound on |fl32(x s) - x s| for |x s| <= qmax (1 + 2^-11) (an fp16 scale
    is at most half an fp16 ulp above qmax / absmax): half an ulp, at most
    2^-24 of the magnitude."""
    return qmax * 2.0 ** -24 * (1 + 2.0 ** -10)


def _tie_example(axis):
    """A (2, 3, 5, 8) input whose element (0, 0, 1, 0) or (0, 0, 0, 1) has a
    float32 product x s on a half-integer while the exact product is not,
    with |x s| > 64 (an error above 0.5 / s by several parts per million)."""
    for x_t, s in f32_tie_pairs(400, 127, seed=99, scale_range=(150.0, 250.0)):
        if abs(fr(x_t) * fr(s)) < 64:
            continue
        a = nearest_f32(Fraction(127) / fr(s))      # absmax whose fp16 scale is s
        if np.float16(np.float32(127) / a) != s or abs(x_t) > a:
            continue
        x = np.zeros((2, 3, 5, 8), np.float32)
        x[0, 0, 0, 0] = a
        x[(0, 0, 1, 0) if axis == "key" else (0, 0, 0, 1)] = x_t
        return x
    raise AssertionError("no tie example found")


def test_key_grid_example(golden):
    g = golden("worked_example_sec03.json")
    scale = np.float32(1.0 / g["k_grid_step"])        # inverse step
    codes = codec.quantize_with_scale(np.array(g["k"], np.float32), scale, qmax=127)
    assert codes.tolist() == [1, 1]
    k_hat = codec.restore(codes, np.float32(scale), dtype=np.float64)
    assert np.allclose(k_hat, g["k_hat"], rtol=0, atol=1e-7)


def test_value_grid_example(golden):
    g = golden("worked_example_sec03.json")
    scale = np.float32(1.0 / g["v_grid_step"])
    codes = codec.quantize_with_scale(np.array(g["v_only_values"], np.float32), scale, qmax=127)
    assert codes.tolist() == [2, 6]
    v_hat = codec.restore(codes, np.float32(scale), dtype=np.float64)
    assert v_hat.tolist() == g["v_hat"]
    w = np.array(g["v_only_weights"])
    assert abs(w @ np.array(g["v_only_values"]) - g["v_only_output_before"]) < 1e-12
    assert abs(w @ v_hat - g["v_only_output_after"]) < 1e-12


def test_round_half_to_even_ties():
    # scale = 7 / 7 = 1 exactly, so every product below is an exact tie or integer.
    x = np.array([7, 2.5, -2.5, 0.5, 1.5, -0.5, 3.5], np.float32).reshape(1, 1, 1, 7)
    codes, scale = codec.quantize_value_per_token(x, qmax=7)
    assert scale.ravel().tolist() == [1.0]
    assert codes.ravel().tolist() == [7, 2, -2, 0, 2, 0, 4]


def test_scale_shapes_follow_the_axes():
    rng = np.random.default_rng(0)
    key = rng.standard_normal((1, 2, 5, 8)).astype(np.float32)
    k_q, k_s = codec.quantize_key_per_channel(key)
    v_q, v_s = codec.quantize_value_per_token(key)
    assert k_q.shape == key.shape and k_s.shape == (1, 2, 1, 8)
    assert v_q.shape == key.shape and v_s.shape == (1, 2, 5, 1)


def test_axes_reduce_over_the_right_dimension():
    # One huge Key token must set every channel's scale; one huge Value
    # channel must set every token's scale -- and nothing else.
    x = np.ones((1, 1, 4, 3), np.float32)
    x[0, 0, 2, :] = 70.0
    _, k_s = codec.quantize_key_per_channel(x, qmax=7)
    assert np.all(k_s == np.float32(7) / np.float32(70))
    _, v_s = codec.quantize_value_per_token(x, qmax=7)
    assert v_s.ravel().tolist() == [7.0, 7.0, np.float32(7) / np.float32(70), 7.0]


def test_rank_is_checked():
    with pytest.raises(ValueError):
        codec.quantize_key_per_channel(np.zeros((2, 3, 4), np.float32))
    with pytest.raises(ValueError):
        codec.quantize_value_per_token(np.zeros((2, 3, 4), np.float32))


@pytest.mark.parametrize("storage", ["fp32", "fp16"])
def test_zero_range_scale_is_finite(storage):
    zeros = np.zeros((1, 1, 3, 4), np.float32)
    k_q, k_s = codec.quantize_key_per_channel(zeros, storage=storage)
    v_q, v_s = codec.quantize_value_per_token(zeros, storage=storage)
    assert np.isfinite(k_s.astype(np.float64)).all() and np.isfinite(v_s.astype(np.float64)).all()
    assert not k_q.any() and not v_q.any()
    assert not codec.restore(k_q, k_s, dtype=np.float64).any()
    if storage == "fp16":
        # 7 / 1e-8 overflows fp16; the stored scale saturates at the largest finite fp16.
        assert k_s.dtype == np.float16 and np.all(k_s == np.float16(65504))


def test_fp16_storage_rounding_and_saturation():
    # Normal range: the stored scale is within half an fp16 ulp (2^-11 relative).
    absmax = np.array([0.5, 1.0, 2.8, 3.3, 29.0, 1000.0], np.float32)
    s16 = codec.scale_from_absmax(absmax, 7, 1e-8, "fp16").astype(np.float64)
    s32 = (np.float32(7) / absmax).astype(np.float64)
    assert np.all(np.abs(s16 - s32) <= s32 * 2.0 ** -11)
    # A tiny range saturates instead of overflowing.
    tiny = codec.scale_from_absmax(np.float32(1e-6), 7, 1e-8, "fp16")
    assert tiny == np.float16(65504)
    # Exactly representable scales are kept exactly.
    assert codec.scale_from_absmax(np.float32(7.0), 7, 1e-8, "fp16") == np.float16(1.0)
    assert codec.scale_from_absmax(np.float32(0.5), 1, 1e-8, "fp16") == np.float16(2.0)


def test_overwritten_scale_scales_old_values():
    # "KV Cache quantization and compression", section 02: codes made with step
    # 0.1 and read back with step 0.2 come back exactly doubled.
    x = np.array([0.3, -0.7, 1.2], np.float32)
    codes = codec.quantize_with_scale(x, np.float32(10.0), qmax=127)
    good = codec.restore(codes, np.float32(10.0), dtype=np.float64)
    bad = codec.restore(codes, np.float32(5.0), dtype=np.float64)
    assert np.array_equal(bad, 2 * good)


@settings(max_examples=60, deadline=None)
@example(x=_tie_example("key"), qmax=127, storage="fp16", axis="key")
@example(x=_tie_example("value"), qmax=127, storage="fp16", axis="value")
@given(
    x=hnp.arrays(np.float32, (2, 3, 5, 8),
                 elements=st.floats(-50, 50, width=32, allow_nan=False)),
    qmax=st.sampled_from([1, 7, 127]),
    storage=st.sampled_from(["fp32", "fp16"]),
    axis=st.sampled_from(["key", "value"]),
)
def test_uniform_quantizer_bounds(x, qmax, storage, axis):
    quant = codec.quantize_key_per_channel if axis == "key" else codec.quantize_value_per_token
    codes, scale = quant(x, qmax=qmax, storage=storage)
    s = np.broadcast_to(scale.astype(np.float64), x.shape)
    assert np.all(np.abs(codes.astype(np.int32)) <= qmax)
    # Half a step of error, plus the float32 rounding of the product x * s
    # (the codes round fl32(x s), not x s), plus float64 rounding in this check.
    err = np.abs(x.astype(np.float64) - codes / s)
    assert np.all(err <= (0.5 + product_slack(qmax)) / s * (1 + 2.0 ** -40) + 1e-30)
    # The element that sets a channel's / token's range lands on +-qmax
    # unless the scale saturated (fp16 storage of a tiny range).
    red = -2 if axis == "key" else -1
    amax = np.abs(x).max(axis=red, keepdims=True)
    is_max = (np.abs(x) == amax) & (amax > 0)
    unsaturated = np.broadcast_to(scale.astype(np.float64) < 65504, x.shape)
    hit = np.abs(codes.astype(np.int32)) == qmax
    assert np.all(hit[is_max & unsaturated])


def test_grouped_over_all_of_head_dim_is_the_per_token_quantizer():
    x = np.random.default_rng(11).standard_normal((2, 3, 17, 64)).astype(np.float32) * 3
    for storage in ("fp32", "fp16"):
        c1, s1 = codec.quantize_grouped_per_token(x, 64, 7, 1e-8, storage)
        c2, s2 = codec.quantize_value_per_token(x, 7, 1e-8, storage)
        assert np.array_equal(c1, c2)
        assert np.array_equal(s1[..., 0, :], s2)


def test_grouped_runs_are_independent_and_bounded():
    """Each run of `group` channels has its own range: scaling one run leaves
    the others' codes unchanged; the run's absmax element reaches +-qmax and
    every element restores within half a step."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, 2, 9, 128)).astype(np.float32)
    c, s = codec.quantize_grouped_per_token(x, 32, 7)
    y = x.copy()
    y[..., 32:64] *= 10
    c2, _ = codec.quantize_grouped_per_token(y, 32, 7)
    keep = np.r_[0:32, 64:128]
    assert np.array_equal(c[..., keep], c2[..., keep])
    runs = np.abs(x).reshape(1, 2, 9, 4, 32)
    hit = np.abs(c.astype(np.int32)).reshape(1, 2, 9, 4, 32) == 7
    assert np.all(hit[runs == runs.max(axis=-1, keepdims=True)])
    xr = codec.restore_grouped_per_token(c, s)
    step = np.repeat(1.0 / s.astype(np.float64)[..., 0], 32, axis=-1)
    assert np.all(np.abs(xr - x) <= (0.5 + product_slack(7)) * step * (1 + 2.0 ** -40))


def test_tie_examples_exceed_half_a_step():
    """The stored examples really sit above 0.5 / s: a bound without the
    product's rounding would fail on a correct quantizer."""
    for axis in ("key", "value"):
        x = _tie_example(axis)
        quant = codec.quantize_key_per_channel if axis == "key" else codec.quantize_value_per_token
        codes, scale = quant(x, qmax=127, storage="fp16")
        s = np.broadcast_to(scale.astype(np.float64), x.shape)
        ratio = (np.abs(x.astype(np.float64) - codes / s) / (0.5 / s)).max()
        assert 1 + 1e-6 < ratio <= 1 + product_slack(127) * 2 * (1 + 2.0 ** -40)


def test_restore_is_the_correctly_rounded_f32_quotient():
    """restore(code, s) in float32 is code / max(s, eps) rounded once to
    binary32 ("KV Cache Quantization Strategies", Step 4 restore: a float
    division by the clamped scale).  The reference is the exact rational
    quotient rounded to nearest-even binary32; restoring through a reciprocal
    (code * (1 / s): two roundings) differs on a share of these pairs."""
    rng = np.random.default_rng(21)
    eps = 1e-8
    s16 = rng.uniform(1e-3, 4000.0, 2000).astype(np.float16)
    s16[:5] = 0.0                                      # below eps: the floor is used
    s32 = (np.float32(7) / rng.uniform(1e-3, 30.0, 2000).astype(np.float32)).astype(np.float32)
    floor = fr(np.float32(eps))
    for scales in (s16, s32):
        codes = rng.integers(-127, 128, scales.size).astype(np.int8)
        got = codec.restore(codes, scales, eps=eps, dtype=np.float32)
        exp = np.array([nearest_f32(Fraction(int(c)) / max(fr(s), floor)) for c, s in zip(codes, scales)],
                       np.float32)
        assert got.dtype == np.float32
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))
        recip = codes.astype(np.float32) * (np.float32(1) / np.maximum(scales.astype(np.float32), np.float32(eps)))
        assert (recip.view(np.uint32) != exp.view(np.uint32)).sum() > scales.size // 20


@pytest.mark.parametrize("qmax", [1, 7, 127])
def test_codes_round_the_f32_product_half_to_even(qmax):
    """code = clamp(rne(fl32(x * s))): the product is rounded to float32 first
    (Step 4 ``_quantize`` multiplies float32 operands), then half-to-even.
    Each pair's exact product lies just off a half-integer that its float32
    rounding lands on, so an exact or float64 product picks the other
    neighbour; the expected code is computed here by exact arithmetic."""
    pairs = f32_tie_pairs(40, max(qmax, 2), seed=qmax)
    pairs = [(x, s) for x, s in pairs if abs(fr(x) * fr(s)) < qmax]
    assert len(pairs) >= (20 if qmax > 1 else 1)
    x = np.array([p[0] for p in pairs], np.float32)
    s = np.array([p[1] for p in pairs], np.float16)
    got = codec.quantize_with_scale(x, s, qmax).tolist()
    exp = [max(-qmax, min(qmax, round_half_even(fr(nearest_f32(fr(a) * fr(b)))))) for a, b in pairs]
    assert got == exp
    assert all(e != round_half_even(fr(a) * fr(b)) for e, (a, b) in zip(exp, pairs))


def test_tie_products_through_the_axis_quantizers():
    """The same ties reached through the scale a range gives: for a token
    row [a, x] (Values) or a channel column (Keys) the stored fp16 scale is s
    and x's code is the half-even rounding of fl32(x s)."""
    for x_t, s in f32_tie_pairs(30, 7, seed=5, scale_range=(2.0, 60.0)):
        a = nearest_f32(Fraction(7) / fr(s))
        if np.float16(np.float32(7) / a) != s or abs(x_t) > a:
            continue
        want = round_half_even(fr(nearest_f32(fr(x_t) * fr(s))))
        row = np.zeros((1, 1, 1, 4), np.float32)
        row[..., 0], row[..., 2] = a, x_t
        codes, scale = codec.quantize_value_per_token(row, 7, 1e-8, "fp16")
        assert scale.ravel()[0] == s and int(codes[0, 0, 0, 2]) == want
        col = np.zeros((1, 1, 3, 2), np.float32)
        col[0, 0, 0, 1], col[0, 0, 2, 1] = a, x_t
        codes, scale = codec.quantize_key_per_channel(col, 7, 1e-8, "fp16")
        assert scale.ravel()[1] == s and int(codes[0, 0, 2, 1]) == want
