"""Byte ledgers of the cache (test infrastructure).

* ``kv_bytes`` -- 2 (K and V) x layers x KV heads x head_dim x positions x
  bytes per element ("KV Cache quantization and compression", section 01
  table; "KV Cache and autoregressive video generation", section 3.3).
* ``quantized_bytes`` -- low-bit codes plus one 2-byte fp16 scale per
  ``scalars_per_scale`` scalars (the former page, section 05).
* ``window_split_bytes`` -- newest ``window`` positions kept at 16 bits, the
  rest at ``bits`` (section 05, "latest 128 positions at 16 bits").
* ``compare`` -- the exercise's ``compare`` ledger ("KV Cache Quantization
  Strategies", Step 4): raw bytes, int8-container bytes, and packed bytes
  ceil(n * bits / 8) plus scale bytes (the page hard-codes bits = 4 via
  (n + 1) // 2; ``bits`` generalises it).

Parity: pinned by tests/test_oracle_layout_ledger.py against the printed budgets
(512 / 256 / 128 / 260 / 132 / 140 MiB, 131072 bytes per token, 52.73 GiB for
432000 tokens).
"""
from __future__ import annotations

import numpy as np

from .codec import quantize_key_per_channel, quantize_value_per_token, restore

MIB = 1 << 20
GIB = 1 << 30


def kv_bytes(layers: int, kv_heads: int, head_dim: int, positions: int, bytes_per_elem: float):
    return 2 * layers * kv_heads * head_dim * positions * bytes_per_elem


def packed_code_bytes(n_codes: int, bits: int) -> int:
    return -(-n_codes * bits // 8)


def quantized_bytes(n_scalars: int, bits: int, scalars_per_scale: int, scale_bytes: int = 2):
    return packed_code_bytes(n_scalars, bits) + (n_scalars // scalars_per_scale) * scale_bytes


def window_split_bytes(layers, kv_heads, head_dim, positions, window, bits):
    """(high-precision window bytes, low-bit code bytes) without scales."""
    hi = kv_bytes(layers, kv_heads, head_dim, window, 2)
    lo = packed_code_bytes(2 * layers * kv_heads * head_dim * (positions - window), bits)
    return hi, lo


def compare(key, value, qmax: int = 7, eps: float = 1e-8, bits: int = 4,
            elem_bytes: int = 4, storage: str = "fp32"):
    key = np.asarray(key, np.float32)
    value = np.asarray(value, np.float32)
    k_q, k_s = quantize_key_per_channel(key, qmax, eps, storage)
    v_q, v_s = quantize_value_per_token(value, qmax, eps, storage)
    k_r = restore(k_q, k_s, eps)
    v_r = restore(v_q, v_s, eps)
    scale_bytes = k_s.size * k_s.itemsize + v_s.size * v_s.itemsize
    return {
        "key_scale_shape": k_s.shape,
        "value_scale_shape": v_s.shape,
        "key_mse": float(np.mean((key - k_r) ** 2)),
        "value_mse": float(np.mean((value - v_r) ** 2)),
        "raw_bytes": (key.size + value.size) * elem_bytes,
        "container_quantized_bytes": k_q.size * k_q.itemsize + v_q.size * v_q.itemsize + scale_bytes,
        "packed_quantized_bytes": packed_code_bytes(k_q.size + v_q.size, bits) + scale_bytes,
    }
