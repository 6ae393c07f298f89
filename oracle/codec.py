"""Oracle codec: KIVI-style asymmetric-axis quantization (test infrastructure).

Source: "KV Cache Quantization Strategies" (page 1), Step 2 (which axis each
of K and V reduces over, and the scale shapes) and the Step 4 reference
solution (``_quantize``, ``restore``, ``quantize_key_per_channel``,
``quantize_value_per_token``).

The page's steps, in its order and notation:

1. absmax = |x| reduced over the token axis (Key, scale [..., 1, head_dim])
   or over head_dim (Value, scale [..., tokens, 1]), keeping the dim;
2. scale = qmax / max(absmax, eps)  -- an *inverse* step: restore divides;
3. codes = clamp(round(float32(x) * scale), -qmax, qmax) in an int8 container,
   where ``round`` is half-to-even (torch.round);
4. restore(codes, scale) = codes / max(scale, eps).

All of steps 1-3 run in float32, as the page's ``x.float()`` does; numpy's
float32 divide and multiply are single IEEE-754 operations, and ``np.rint`` is
round-half-to-even.

Scale storage.  The page keeps ``scale`` in float32 ("fp32" storage, used to
replay its own tests).  The library stores scales as fp16, which the page's
float32 ``qmax / eps`` (7e8) would overflow to +inf; the reading taken is to
clamp the float32 scale at 65504 (the largest finite fp16) and then round to
fp16 half-to-even, and to compute the codes with the *stored* fp16 scale so
that restore uses exactly the scale the codes were made with.  Clamping only
lowers a scale, so no element clips beyond half a step.

Same-axis grouping (``quantize_grouped_per_token``): the Step 2 table's
third row, one fixed-size local group, as in section 5.1's setting (groups
of 64 along head_dim for both K and V): steps 1-4 with the absmax taken over
each run of ``group`` consecutive channels of one token.

Parity: pinned by tests/test_oracle_codec.py (worked grid examples of "KV
Cache quantization and compression" section 03, the round-half-even tie
vector, the all-zero range contract, the per-element error bound, fp16
conversion against numpy's own float16 cast; grouping over the whole of
head_dim equals the per-token quantizer).
"""
from __future__ import annotations

import numpy as np

FP16_MAX = np.float32(65504.0)


def quantize_with_scale(x, scale, qmax: int) -> np.ndarray:
    """clamp(round_half_even(float32(x) * float32(scale)), -qmax, qmax) as int8."""
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(scale).astype(np.float32)
    prod = np.multiply(x32, s32, dtype=np.float32)
    return np.clip(np.rint(prod), -qmax, qmax).astype(np.int8)


def scale_from_absmax(absmax, qmax: int, eps: float, storage: str = "fp32") -> np.ndarray:
    """qmax / max(absmax, eps) in float32; optionally stored as saturated fp16."""
    a = np.maximum(np.asarray(absmax, dtype=np.float32), np.float32(eps))
    s32 = np.divide(np.float32(qmax), a, dtype=np.float32)
    if storage == "fp32":
        return s32
    if storage == "fp16":
        return np.minimum(s32, FP16_MAX).astype(np.float16)
    raise ValueError(f"unknown scale storage {storage!r}")


def _check4(x, what):
    if np.ndim(x) != 4:
        raise ValueError(f"{what}: expected a 4-D [batch, heads, tokens, head_dim] array, got {np.ndim(x)}-D")


def quantize_key_per_channel(key, qmax: int = 7, eps: float = 1e-8, storage: str = "fp32"):
    """Per-channel Key codes: absmax over the token axis, scale [..., 1, head_dim]."""
    _check4(key, "key")
    x = np.asarray(key, dtype=np.float32)
    absmax = np.abs(x).max(axis=-2, keepdims=True)
    scale = scale_from_absmax(absmax, qmax, eps, storage)
    return quantize_with_scale(x, scale, qmax), scale


def quantize_value_per_token(value, qmax: int = 7, eps: float = 1e-8, storage: str = "fp32"):
    """Per-token Value codes: absmax over head_dim, scale [..., tokens, 1]."""
    _check4(value, "value")
    x = np.asarray(value, dtype=np.float32)
    absmax = np.abs(x).max(axis=-1, keepdims=True)
    scale = scale_from_absmax(absmax, qmax, eps, storage)
    return quantize_with_scale(x, scale, qmax), scale


def restore(codes, scale, eps: float = 1e-8, dtype=None) -> np.ndarray:
    """codes / max(scale, eps), computed in ``dtype`` (default: the scale's dtype)."""
    s = np.asarray(scale)
    dt = np.dtype(dtype) if dtype is not None else s.dtype
    floor = np.asarray(np.float32(eps)).astype(dt)
    return np.asarray(codes).astype(dt) / np.maximum(s.astype(dt), floor)


def quantize_grouped_per_token(x, group: int, qmax: int = 7, eps: float = 1e-8, storage: str = "fp32"):
    """Same-axis codes: absmax over each run of ``group`` consecutive channels
    of a token; scale [..., tokens, head_dim // group, 1]."""
    _check4(x, "x")
    a = np.asarray(x, dtype=np.float32)
    B, H, T, D = a.shape
    if group < 1 or D % group:
        raise ValueError("group must divide head_dim")
    runs = a.reshape(B, H, T, D // group, group)
    absmax = np.abs(runs).max(axis=-1, keepdims=True)
    scale = scale_from_absmax(absmax, qmax, eps, storage)
    return quantize_with_scale(runs, scale, qmax).reshape(B, H, T, D), scale


def restore_grouped_per_token(codes, scale, eps: float = 1e-8, dtype=np.float64) -> np.ndarray:
    """codes / max(scale, eps) for ``quantize_grouped_per_token`` codes."""
    c = np.asarray(codes)
    B, H, T, D = c.shape
    G = np.shape(scale)[-2]
    runs = c.reshape(B, H, T, G, D // G)
    return restore(runs, scale, eps, dtype).reshape(B, H, T, D)
