"""Pins for the oracle attention (decode and block).

Fixed by: the worked numbers of "KV Cache quantization and compression"
section 03 (tests/golden/worked_example_sec03.json), and closed forms that
follow from the definition softmax(sigma q K^T + M) V -- q = 0 gives the
plain mean of the visible values, one visible token gives its value, two
tokens give a logistic blend, KV-head replication makes query head h read
KV head h // g, and the causal mask makes row i see N + i + 1 tokens.
"""
import numpy as np
import pytest

from oracle import attention
from oracle.cache import KVQuantizationStrategies


def test_worked_example(golden):
    g = golden("worked_example_sec03.json")
    q = np.array([[g["q"]]])
    K = np.array(g["k"])[:, None]
    out = attention.attention_rows(q, K, np.array(g["v"])[:, None], g["sigma"])
    assert abs(out[0, 0] - g["output"]) < 0.5 * 10.0 ** -g["printed_decimals"]
    # With V = identity the output row is the softmax itself.
    p = attention.attention_rows(q, K, np.eye(2), g["sigma"])[0]
    assert np.all(np.abs(p - g["softmax"]) < 0.5 * 10.0 ** -g["printed_decimals"])
    # K on the 0.2 grid: equal scores, equal weights, output 2.0.
    out = attention.attention_rows(q, np.array(g["k_hat"])[:, None], np.array(g["v"])[:, None], 1.0)
    assert abs(out[0, 0] - g["k_grid_output"]) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((7, 5))
    V = rng.standard_normal((7, 5))
    # q = 0: uniform weights over the visible tokens.
    out = attention.attention_rows(np.zeros((3, 5)), K, V, 0.3, visible=[1, 4, 7])
    assert np.allclose(out[0], V[0], atol=1e-14)
    assert np.allclose(out[1], V[:4].mean(0), atol=1e-14)
    assert np.allclose(out[2], V.mean(0), atol=1e-14)
    # Two tokens: v1 + (v2 - v1) * logistic(sigma * q.(k2 - k1)).
    q = rng.standard_normal((1, 5))
    sig = 0.7
    w2 = 1.0 / (1.0 + np.exp(-sig * (q[0] @ (K[1] - K[0]))))
    out = attention.attention_rows(q, K[:2], V[:2], sig)
    assert np.allclose(out[0], V[0] + (V[1] - V[0]) * w2, atol=1e-14)
    # Large logits stay finite (max subtraction).
    out = attention.attention_rows(1e3 * np.ones((1, 5)), K, V, 1.0)
    assert np.isfinite(out).all()


def _exact_grid_state(rng, B, H, T, D, R, G, qmax=7):
    """K/V whose values sit exactly on each segment's grid, so restore is exact."""
    s = KVQuantizationStrategies(qmax=qmax, scale_storage="fp16", group=G)
    # Values k = code / 2^e with the code at +-qmax somewhere in each channel /
    # token make absmax = qmax / 2^e and the scale exactly 2^e (no rounding).
    # Each group of G tokens gets its own power-of-two step, so a token read
    # with another segment's Key scale would come back wrong.
    codes = rng.integers(-qmax, qmax + 1, size=(B, H, T, D))
    codes[..., :, 0] = qmax          # every V token reaches qmax
    step = np.full(T, 0.25)
    if G:
        for j, start in enumerate(range(0, T, G)):
            codes[..., start, :] = qmax  # every K channel reaches qmax in every group
            step[start:start + G] = 2.0 ** -(1 + j % 3)
    else:
        codes[..., 0, :] = qmax
    k = (codes * step[:, None]).astype(np.float32)
    v = (codes / 2.0).astype(np.float32)
    return s.append_and_partition(None, k, v, R), k, v


@pytest.mark.parametrize("G", [0, 4])
def test_decode_assembles_prefix_then_tail(G):
    rng = np.random.default_rng(2)
    B, H, T, D, g = 2, 2, 13, 4, 3
    st_, k, v = _exact_grid_state(rng, B, H, T, D, R=3, G=G)
    assert st_["quantized_tokens"] > 0
    q = rng.standard_normal((B, H * g, D))
    out = attention.decode_attention(st_, q, sigma=0.5)
    for b in range(B):
        for h in range(H * g):
            ref = attention.attention_rows(q[b, h][None], k[b, h // g], v[b, h // g], 0.5)
            assert np.allclose(out[b, h], ref[0], atol=1e-12)


def test_gqa_head_mapping():
    B, H, T, D, g = 1, 3, 5, 4, 4
    v = np.zeros((B, H, T, D), np.float32)
    for h in range(H):
        v[:, h] = h + 1
    k = np.random.default_rng(3).standard_normal((B, H, T, D)).astype(np.float32)
    st_ = KVQuantizationStrategies(group=0).append_and_partition(None, k, v, residual_length=T)
    q = np.random.default_rng(4).standard_normal((B, H * g, D))
    out = attention.decode_attention(st_, q, sigma=1.0)
    for h in range(H * g):
        assert np.allclose(out[0, h], h // g + 1, atol=1e-12)


def test_block_causal_visibility():
    rng = np.random.default_rng(5)
    B, H, N, D, g, Tq = 1, 2, 6, 4, 2, 5
    k = rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    st_ = KVQuantizationStrategies(group=0).append_and_partition(None, k, v, residual_length=N)
    kb = rng.standard_normal((B, Tq, H, D))
    vb = rng.standard_normal((B, Tq, H, D))
    q = np.zeros((B, Tq, H * g, D))
    out = attention.block_attention(st_, q, kb, vb, sigma=1.0)
    for i in range(Tq):
        for h in range(H * g):
            vis = np.concatenate((v[0, h // g], vb[0, :i + 1, h // g]))
            assert np.allclose(out[0, i, h], vis.mean(0), atol=1e-12)
    # A one-query block equals decode after appending that token.
    q1 = rng.standard_normal((B, 1, H * g, D))
    blk = attention.block_attention(st_, q1, kb[:, :1], vb[:, :1], sigma=0.4)
    st2 = KVQuantizationStrategies(group=0).append_and_partition(
        st_, kb[:, :1].transpose(0, 2, 1, 3), vb[:, :1].transpose(0, 2, 1, 3), residual_length=N + 1)
    dec = attention.decode_attention(st2, q1[:, 0], sigma=0.4)
    assert np.allclose(blk[:, 0], dec, atol=1e-6)


def test_frame_mask_matches_the_video_figure():
    """"KV Cache and autoregressive video generation", section 6.3 figure:
    5 frames of 12 tokens; a frame sees itself and every earlier frame (the
    upper-right blocks are empty, the diagonal blocks full)."""
    m = attention.block_mask(0, np.arange(60), 60, frame_tokens=12)
    expect = np.kron(np.tril(np.ones((5, 5), bool)), np.ones((12, 12), bool))
    assert np.array_equal(m, expect)
    # frames of one token are the token-causal mask
    assert np.array_equal(attention.block_mask(0, np.arange(7), 7, 1), np.tril(np.ones((7, 7), bool)))
    # cached tokens are always visible
    assert attention.block_mask(9, np.arange(3), 3, 2)[:, :9].all()


def test_frame_mask_with_a_partly_cached_frame():
    """N = 5 cached tokens, frames of 4: positions 5..7 close frame 1 (they see
    block tokens 0..2), positions 8..11 form frame 2 (block tokens 0..6)."""
    m = attention.block_mask(5, np.arange(7), 7, frame_tokens=4)
    assert m[:, :5].all()
    assert [int(r[5:].sum()) for r in m] == [3, 3, 3, 7, 7, 7, 7]


def test_block_frames_bidirectional_inside_a_frame():
    """One frame spanning the whole block: every query sees every block token,
    so q = 0 returns the mean of all cached and block values for every row;
    frame_tokens = 1 keeps the token-causal result."""
    rng = np.random.default_rng(6)
    B, H, N, D, g, Tq = 1, 2, 8, 4, 2, 6
    k = rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    st_ = KVQuantizationStrategies(group=0).append_and_partition(None, k, v, residual_length=N)
    kb = rng.standard_normal((B, Tq, H, D))
    vb = rng.standard_normal((B, Tq, H, D))
    q0 = np.zeros((B, Tq, H * g, D))
    out = attention.block_attention(st_, q0, kb, vb, sigma=1.0, frame_tokens=N + Tq)
    for h in range(H * g):
        allv = np.concatenate((v[0, h // g], vb[0, :, h // g]))
        assert np.allclose(out[0, :, h], allv.mean(0), atol=1e-12)
    q = rng.standard_normal((B, Tq, H * g, D))
    a = attention.block_attention(st_, q, kb, vb, sigma=0.5)
    b = attention.block_attention(st_, q, kb, vb, sigma=0.5, frame_tokens=1)
    assert np.array_equal(a, b)


def test_axis_study_outlier_channels_favour_per_channel_keys():
    """Keys with channels ten times larger (the synthetic workloads' outliers):
    a per-channel Key range restores the other channels far better than runs
    of 64 channels that contain an outlier; Values are per token in both."""
    from oracle import axis_study
    rng = np.random.default_rng(13)
    B, H, T, D = 1, 2, 256, 128
    k = rng.standard_normal((B, H, T, D))
    k[..., [5, 70]] *= 10
    v = rng.standard_normal((B, H, T, D))
    q = rng.standard_normal((B, 4, D))
    r = axis_study.compare(k, v, q, qmax=7, segment=128, group=64)
    assert r["kivi"]["k_rms"] < 0.6 * r["same_axis"]["k_rms"]
    assert r["kivi"]["attn_rms"] < r["same_axis"]["attn_rms"]
    # with one scale over all of head_dim and no outliers, Values are the same in both
    r0 = axis_study.compare(rng.standard_normal((B, H, T, D)), v, q, qmax=7, segment=128, group=128)
    assert abs(r0["kivi"]["v_rms"] - r0["same_axis"]["v_rms"]) < 1e-12
