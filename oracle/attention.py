"""Oracle attention over a quantized cache, in float64 (test infrastructure).

Definition ("KV Cache and autoregressive video generation", section 3.1):
    Attn(Q, K, V) = softmax(Q K^T * sigma + M) V,
with the causal mask M_ij = 0 for j <= i and -inf otherwise, and the
incremental-decode form o_t = sum_{j<=t} softmax_j(q_t k_j^T * sigma) v_j.
Grouped-query attention repeats each KV head g = Hq / Hkv times, so query head
h reads KV head floor(h / g) (section 04, ``attn_full`` / ``attn_step``).

The cache supplies, per (batch, KV head), the restored quantized prefix
(codes / max(scale, eps), "KV Cache Quantization Strategies" Step 4
``restore``, with the scale of the token's segment and channel for KIVI Keys
or of the token's run of channels in same-axis mode) followed by the
high-precision tail; for decode the newest
token has already been appended, so it is visible ("KV Cache quantization
and compression", section 02 pseudo-code: append, then attention).

Block attention: query i of a block of Tq queries sits at absolute position
N + i, after the N cached tokens; it sees all N cached tokens and the block's
own (not yet appended) tokens 0..i.  With frames of F tokens ("KV Cache and
autoregressive video generation", section 6.3: bidirectional inside a frame,
causal across frames) it sees the block tokens j whose frame
floor((N + j) / F) is not later than its own, floor((N + i) / F); F = 1 is
the token-causal mask.

``sigma`` is a parameter: 1/sqrt(head_dim) in the workloads; the scalar worked
example of "KV Cache quantization and compression" section 03 uses 1.

Everything is the plain definition: one matrix product for the scores, max
subtraction, exp, normalisation, one matrix product with V.

Parity: pinned by tests/test_oracle_attention.py (the section 03 worked
numbers, closed forms: q = 0 gives the mean of the visible values, one token
gives its value, two tokens give a sigmoid blend; GQA head mapping; causal
visibility count).
"""
from __future__ import annotations

import numpy as np

from .cache import key_scales, segment_of_tokens, stacked_codes, value_scales
from .codec import restore, restore_grouped_per_token


def attention_rows(q_rows, K, V, sigma: float, visible=None, mask=None) -> np.ndarray:
    """softmax(sigma * q K^T) V for each row of q, row i seeing K[:visible[i]],
    or the keys where mask[i] is True."""
    q = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    scores = sigma * (q @ K.T)
    if visible is not None:
        visible = np.asarray(visible).reshape(-1, 1)
        scores = np.where(np.arange(K.shape[0])[None, :] < visible, scores, -np.inf)
    if mask is not None:
        scores = np.where(np.asarray(mask, bool), scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V


class _Joined:
    """The state's segments joined once (codes, scales, token -> segment map)."""

    def __init__(self, state):
        self.k_codes = stacked_codes(state, "key")
        self.v_codes = stacked_codes(state, "value")
        self.k_scales = key_scales(state)
        self.v_scales = value_scales(state)
        self.seg = segment_of_tokens(state)
        self.axis_group = state.get("axis_group", 0)


def restored_cache(state, b: int, h: int, eps: float = 1e-8, joined=None):
    """(K_hat, V_hat) for one (batch, KV head): restored prefix, then the tail, float64."""
    j = joined if joined is not None else _Joined(state)
    k_codes = j.k_codes[b, h]                            # [Nq, D]
    v_codes = j.v_codes[b, h]
    if j.axis_group:                                     # same-axis: [Nq, runs] scales for both
        k_hat = restore_grouped_per_token(k_codes[None, None], j.k_scales[b, h][None, None, :, :, None],
                                          eps, np.float64)[0, 0]
        v_hat = restore_grouped_per_token(v_codes[None, None], j.v_scales[b, h][None, None, :, :, None],
                                          eps, np.float64)[0, 0]
    else:
        k_scale = j.k_scales[b, h][j.seg]                # [Nq, D]: the token's segment row
        v_scale = j.v_scales[b, h][:, None]              # [Nq, 1]
        k_hat = restore(k_codes, k_scale, eps, np.float64)
        v_hat = restore(v_codes, v_scale, eps, np.float64)
    k_tail = np.asarray(state["key_residual"][b, h], np.float64)
    v_tail = np.asarray(state["value_residual"][b, h], np.float64)
    return np.concatenate((k_hat, k_tail)), np.concatenate((v_hat, v_tail))


def decode_attention(state, q, sigma: float, eps: float = 1e-8, units=None) -> np.ndarray:
    """Single-query GQA attention over the whole cache.  q: [B, Hq, D] -> [B, Hq, D].

    ``units`` optionally restricts the work to a list of (b, kv_head) pairs
    (other outputs stay NaN); it exists to time bounded samples.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = state["key_residual"].shape[1]
    if Hq % Hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    g = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    joined = _Joined(state)
    for b, h in todo:
        K, V = restored_cache(state, b, h, eps, joined)
        out[b, h * g:(h + 1) * g] = attention_rows(q[b, h * g:(h + 1) * g], K, V, sigma)
    return out


def block_mask(n_cached: int, rows, tq: int, frame_tokens: int = 1) -> np.ndarray:
    """Visibility [len(rows), n_cached + tq] of block attention: every cached
    token, and block token j for query i iff floor((N + j) / F) <= floor((N + i) / F)."""
    rows = np.asarray(rows)
    frame_q = (n_cached + rows) // frame_tokens
    frame_k = (n_cached + np.arange(tq)) // frame_tokens
    own = frame_k[None, :] <= frame_q[:, None]
    return np.concatenate((np.ones((rows.size, n_cached), bool), own), axis=1)


def block_attention(state, q, k_blk, v_blk, sigma: float, eps: float = 1e-8,
                    rows=None, heads=None, frame_tokens: int = 1) -> np.ndarray:
    """Block attention (causal across frames of ``frame_tokens`` positions,
    bidirectional inside one; 1 = token-causal).  q: [B, Tq, Hq, D];
    k_blk, v_blk: [B, Tq, Hkv, D].

    Returns [B, Tq, Hq, D]; with ``rows``/``heads`` only those query rows /
    query heads are computed (the others stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Tq, Hq, D = q.shape
    Hkv = np.shape(k_blk)[2]
    g = Hq // Hkv
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    heads = range(Hq) if heads is None else heads
    out = np.full((B, Tq, Hq, D), np.nan)
    joined = _Joined(state)
    for b in range(B):
        for kh in sorted({h // g for h in heads}):
            K, V = restored_cache(state, b, kh, eps, joined)
            n_cached = K.shape[0]
            K_all = np.concatenate((K, np.asarray(k_blk[b, :, kh], np.float64)))
            V_all = np.concatenate((V, np.asarray(v_blk[b, :, kh], np.float64)))
            mask = block_mask(n_cached, rows, Tq, frame_tokens)
            for h in heads:
                if h // g != kh:
                    continue
                out[b, rows, h] = attention_rows(q[b, rows, h], K_all, V_all, sigma, mask=mask)
    return out
