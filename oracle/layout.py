"""The library's packed byte layout, written out from its specification.

The pages fix no packing: the exercise keeps 4-bit codes in an int8
container and counts packed bytes as (n + 1) // 2 ("KV Cache Quantization
Strategies", Step 4 ``compare``).  The library packs b-bit codes (b = 8, 4
or 2) as b-bit two's-complement fields, lowest field in the lowest bits, and
tiles each (batch, KV head) stream in 64-token tiles.  This module is an
independent statement of that specification, used to build the bytes the
device buffers must hold; it shares nothing with the library.

Per (batch, KV head) stream, with W = head_dim * b / 8 bytes per token row
(a multiple of 16) and capacity C tokens (a multiple of 64):

* Key codes   -- byte offset of token t, channel c:
      (t // 64) * 64 * W + (r // 16) * 1024 + (t % 64) * 16 + (r % 16),
  with r = (c * b) // 8, field at bit (c * b) % 8.  A 64-token tile is
  W / 16 chunks; chunk j holds bytes 16j..16j+15 of every token's row,
  token after token.
* Value codes -- byte offset of token t, channel c:
      (t // 64) * 64 * W + c * 8 * b + ((t % 64) * b) // 8,
  field at bit ((t % 64) * b) % 8.  A 64-token tile is stored channel after
  channel, each channel packing its 64 tokens.
* Key scales  -- fp16 [batch, heads, max_segments, head_dim]: one row per
  segment (segment k covers tokens [kG, (k+1)G) when G > 0).
* Value scales -- fp16 [batch, heads, C]: one per quantized token.
* Tail ring   -- [batch, heads, ring, head_dim] in the K/V dtype; the tail
  token at absolute position p lives in slot p % ring, with
  ring = R + G (G > 0) or R (G = 0).

Parity: pinned by tests/test_oracle_layout_ledger.py (hand-written bytes for small
cases, read straight off the formulas above).
"""
from __future__ import annotations

import numpy as np

TILE = 64


def row_bytes(head_dim: int, bits: int) -> int:
    w = head_dim * bits // 8
    if head_dim * bits % 128:
        raise ValueError("head_dim * bits must be a multiple of 128")
    return w


def ring_slots(residual: int, group: int) -> int:
    return residual + group if group > 0 else residual


def _fields(codes: np.ndarray, bits: int) -> np.ndarray:
    """Two's-complement b-bit field of each code, as uint8."""
    return (codes.astype(np.int16) & ((1 << bits) - 1)).astype(np.uint8)


def pack_k_stream(codes, bits: int, capacity: int) -> np.ndarray:
    """Key codes [T, D] of one stream -> capacity * W bytes."""
    codes = np.asarray(codes, dtype=np.int8)
    T, D = codes.shape
    W = row_bytes(D, bits)
    out = np.zeros(capacity * W, dtype=np.uint8)
    t = np.arange(T)[:, None]
    c = np.arange(D)[None, :]
    r = (c * bits) // 8
    off = (t // TILE) * TILE * W + (r // 16) * 1024 + (t % TILE) * 16 + (r % 16)
    shift = (c * bits) % 8
    vals = (_fields(codes, bits).astype(np.uint16) << shift).astype(np.uint8)
    np.bitwise_or.at(out, np.broadcast_to(off, (T, D)).ravel(), vals.ravel())
    return out


def pack_v_stream(codes, bits: int, capacity: int) -> np.ndarray:
    """Value codes [T, D] of one stream -> capacity * W bytes."""
    codes = np.asarray(codes, dtype=np.int8)
    T, D = codes.shape
    W = row_bytes(D, bits)
    out = np.zeros(capacity * W, dtype=np.uint8)
    t = np.arange(T)[:, None]
    c = np.arange(D)[None, :]
    i = t % TILE
    off = (t // TILE) * TILE * W + c * 8 * bits + (i * bits) // 8
    shift = np.broadcast_to((i * bits) % 8, (T, D))
    vals = (_fields(codes, bits).astype(np.uint16) << shift).astype(np.uint8)
    np.bitwise_or.at(out, np.broadcast_to(off, (T, D)).ravel(), vals.ravel())
    return out


def pack_cache(codes, bits: int, capacity: int, which: str) -> np.ndarray:
    """codes [B, H, T, D] -> uint8 [B, H, capacity * W] in the K or V layout."""
    codes = np.asarray(codes)
    B, H, T, D = codes.shape
    pack = pack_k_stream if which == "key" else pack_v_stream
    out = np.zeros((B, H, capacity * row_bytes(D, bits)), np.uint8)
    for b in range(B):
        for h in range(H):
            out[b, h] = pack(codes[b, h], bits, capacity)
    return out


def ring_positions(quantized: int, tail: int, ring: int) -> np.ndarray:
    """Ring slot of each tail token, oldest first."""
    return (quantized + np.arange(tail)) % ring
