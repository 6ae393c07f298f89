"""Pins for the oracle's append / residual window / flush state machine.

The first group replays the contracts of "KV Cache Quantization Strategies"
Step 4 tests in the page's literal mode (float32 scales, one segment per
flush).  The second checks hand-derived token counts for the five workloads
(tests/golden/workload_counts.json).  The third checks invariants: token
conservation, only whole groups flushed, the newest tokens stay high
precision, and earlier segments are never rewritten.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.cache import KVQuantizationStrategies, segment_of_tokens, stacked_codes


def randn(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_append_state_contract():
    s = KVQuantizationStrategies()
    st_ = s.append_and_partition(None, randn(1, 2, 3, 8), randn(1, 2, 3, 8, seed=1), 4)
    st_ = s.append_and_partition(st_, randn(1, 2, 2, 8, seed=2), randn(1, 2, 2, 8, seed=3), 4)
    assert st_["total_tokens"] == 5
    assert st_["quantized_tokens"] + st_["key_residual"].shape[-2] == 5
    assert st_["quantized_tokens"] + st_["value_residual"].shape[-2] == 5


def test_residual_window_partition_contract():
    s = KVQuantizationStrategies()
    st_ = s.append_and_partition(None, randn(1, 2, 3, 8), randn(1, 2, 3, 8, seed=1), 2)
    st_ = s.append_and_partition(st_, randn(1, 2, 2, 8, seed=2), randn(1, 2, 2, 8, seed=3), 2)
    assert st_["quantized_tokens"] == 3
    assert sum(seg.shape[-2] for seg in st_["key_q_segments"]) == 3
    assert st_["key_residual"].shape[-2] == 2 and st_["value_residual"].shape[-2] == 2


def test_previous_quantized_segments_are_not_rewritten():
    s = KVQuantizationStrategies()
    st_ = s.append_and_partition(None, randn(1, 1, 3, 4), randn(1, 1, 3, 4, seed=1), 2)
    first = st_["key_q_segments"][0].copy()
    st_ = s.append_and_partition(st_, randn(1, 1, 2, 4, seed=2), randn(1, 1, 2, 4, seed=3), 2)
    assert len(st_["key_q_segments"]) == 2
    assert np.array_equal(st_["key_q_segments"][0], first)
    assert st_["flushed_tokens"] == 2


def test_window_without_overflow_contract():
    s = KVQuantizationStrategies()
    st_ = s.append_and_partition(None, randn(1, 1, 1, 4), randn(1, 1, 1, 4, seed=1), 4)
    st_ = s.append_and_partition(st_, randn(1, 1, 1, 4, seed=2), randn(1, 1, 1, 4, seed=3), 4)
    assert st_["quantized_tokens"] == 0 and st_["flushed_tokens"] == 0
    assert st_["key_residual"].shape[-2] == 2


def test_validation_errors():
    s = KVQuantizationStrategies()
    with pytest.raises(ValueError):
        s.append_and_partition(None, randn(1, 1, 1, 4), randn(1, 1, 1, 4), 0)
    with pytest.raises(ValueError):
        s.append_and_partition(None, randn(1, 1, 4), randn(1, 1, 4), 2)
    with pytest.raises(ValueError):
        s.append_and_partition(None, randn(1, 1, 2, 4), randn(1, 1, 3, 4), 2)


def test_flushed_tokens_are_the_oldest_and_tail_is_verbatim():
    s = KVQuantizationStrategies(group=0)
    k = randn(1, 1, 10, 4)
    st_ = s.append_and_partition(None, k[:, :, :6], k[:, :, :6], 3)
    st_ = s.append_and_partition(st_, k[:, :, 6:], k[:, :, 6:], 3)
    # tail = the 3 newest tokens, bit-for-bit
    assert np.array_equal(st_["key_residual"], k[:, :, 7:])
    # quantized prefix = tokens 0..6 in order: re-quantizing each segment's
    # source tokens by the page's rule gives the stored codes.
    assert st_["segment_starts"] == [0, 3]
    seg0, _ = s.quantize_key_per_channel(k[:, :, 0:3])
    seg1, _ = s.quantize_key_per_channel(k[:, :, 3:7])
    assert np.array_equal(st_["key_q_segments"][0], seg0)
    assert np.array_equal(st_["key_q_segments"][1], seg1)


def _run_counts(R, G, sizes):
    s = KVQuantizationStrategies(qmax=7, scale_storage="fp16", group=G)
    st_ = None
    flushes = 0
    for n in sizes:
        x = np.zeros((1, 1, n, 128 if G else 16), np.float32)
        st_ = s.append_and_partition(st_, x, x, R)
        flushes += st_["flushed_tokens"] > 0
    return st_, flushes


@pytest.mark.parametrize("name", ["tiny", "llama3", "append", "video", "long"])
def test_workload_counts(golden, name):
    g = golden("workload_counts.json")[name]
    st_, _ = _run_counts(g["R"], g["G"], [g["prefill"]])
    assert [st_["quantized_tokens"], st_["total_tokens"] - st_["quantized_tokens"],
            len(st_["key_q_segments"])] == g["after_prefill"]
    if "steps" in g:
        st_, flushes = _run_counts(g["R"], g["G"], [g["prefill"]] + [g["step_tokens"]] * g["steps"])
        assert [st_["quantized_tokens"], st_["total_tokens"] - st_["quantized_tokens"],
                len(st_["key_q_segments"])] == g["after_steps"]
        if "flush_events" in g:
            assert flushes - 1 == g["flush_events"]


@settings(max_examples=40, deadline=None)
@given(
    R=st.integers(1, 9),
    G=st.sampled_from([0, 1, 4, 8]),
    sizes=st.lists(st.integers(0, 13), min_size=1, max_size=8),
)
def test_token_conservation_and_append_only(R, G, sizes):
    s = KVQuantizationStrategies(qmax=7, scale_storage="fp16", group=G)
    rng = np.random.default_rng(len(sizes))
    st_ = None
    total = 0
    history = []
    for n in sizes:
        k = rng.standard_normal((1, 2, n, 4)).astype(np.float32)
        v = rng.standard_normal((1, 2, n, 4)).astype(np.float32)
        st_ = s.append_and_partition(st_, k, v, R)
        total += n
        nq, nt = st_["quantized_tokens"], st_["key_residual"].shape[-2]
        assert nq + nt == total == st_["total_tokens"]
        if G:
            assert nq % G == 0 and nt <= R + G - 1
            assert nt >= min(total, R)
        else:
            assert nt == min(total, R)
        # earlier segments are byte-identical across later appends
        for i, (kq, ks) in enumerate(history):
            assert np.array_equal(st_["key_q_segments"][i], kq)
            assert np.array_equal(st_["key_scale_segments"][i], ks)
        history = [(a.copy(), b.copy()) for a, b in
                   zip(st_["key_q_segments"], st_["key_scale_segments"])]
        assert stacked_codes(st_, "key").shape[-2] == nq
        assert len(segment_of_tokens(st_)) == nq
