"""Seeded synthetic workloads for the quantized KV cache.

This module only draws random numbers and casts them to the storage dtype the
workload names.  It holds none of the quantization or attention arithmetic,
so both the CPU oracle (``oracle/``) and the HIP library's tests and
benchmark can consume the very same bytes from it.

Workload shapes follow the pages: the Llama-3-8B attention geometry (32 query
heads, 8 KV heads, head_dim 128; "KV Cache and autoregressive video
generation", section 3.3 and the appendix's ``LLAMA3_8B`` config) and the
5-second video token count of 30 frames x 14400 = 432000 tokens (same page,
section 01).  The tiny case follows the teaching shape of the
"KV Cache Quantization Strategies" exercise, Step 2.

Value distributions: K, V and Q are standard normals drawn as float32 from
``numpy.random.default_rng(seed)``; a few K channels (the same channels for
every batch row and head) are multiplied by 10 to model the per-channel
outliers that motivate per-channel Key scales.  Draw order is fixed:
outlier channel indices first, then K, then V, then Q.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    code_bits: int
    qmax: int
    residual: int
    group: int              # 0 = one segment per flush (overflow-only)
    kv_dtype: str           # "bf16" or "f32"
    seed: int = 0
    outlier_channels: Optional[Sequence[int]] = None  # fixed channels, else drawn
    n_outliers: int = 4
    outlier_gain: float = 10.0
    prefill: int = 0        # tokens appended before the measured phase
    steps: int = 0          # measured appends / decode steps
    step_tokens: int = 1    # tokens per measured append
    block_q: int = 0        # query block length for block attention
    layers: int = 1         # independent caches run back to back


# The five workloads.  Names describe the workload, with its sizes.
TINY = Workload(
    name="tiny_b1_h2_d16_int8c_q7_r8", batch=1, kv_heads=2, q_heads=2, head_dim=16,
    code_bits=8, qmax=7, residual=8, group=0, kv_dtype="f32", seed=0,
    outlier_channels=(3,), prefill=64, steps=16, step_tokens=1)

LLAMA3_DECODE = Workload(
    name="llama3_8b_decode_b8_ctx4096_int4", batch=8, kv_heads=8, q_heads=32, head_dim=128,
    code_bits=4, qmax=7, residual=128, group=128, kv_dtype="bf16", seed=0,
    prefill=4096, steps=1, step_tokens=1)

LONG_CONTEXT = Workload(
    name="long_decode_b1_ctx131072_int4_x32", batch=1, kv_heads=8, q_heads=32, head_dim=128,
    code_bits=4, qmax=7, residual=128, group=128, kv_dtype="bf16", seed=0,
    prefill=131072, steps=1, step_tokens=1, layers=32)

APPEND_INT8 = Workload(
    name="append_b16_ctx4096_plus2048x16_int8", batch=16, kv_heads=8, q_heads=8, head_dim=128,
    code_bits=8, qmax=127, residual=128, group=128, kv_dtype="bf16", seed=0,
    prefill=4096, steps=128, step_tokens=16)

APPEND_INT4 = dataclasses.replace(
    APPEND_INT8, name="append_b16_ctx4096_plus2048x16_int4", code_bits=4, qmax=7)

VIDEO_BLOCK = Workload(
    name="video_block_ctx432000_int2_tq1024", batch=1, kv_heads=8, q_heads=32, head_dim=128,
    code_bits=2, qmax=1, residual=128, group=128, kv_dtype="bf16", seed=0,
    prefill=432000, block_q=1024)

WORKLOADS = {w.name: w for w in (TINY, LLAMA3_DECODE, LONG_CONTEXT, APPEND_INT8,
                                  APPEND_INT4, VIDEO_BLOCK)}


def _to_storage(x: np.ndarray, kv_dtype: str) -> torch.Tensor:
    """Cast float32 samples to the storage dtype (bf16 uses torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if kv_dtype == "bf16":
        return t.to(torch.bfloat16)
    if kv_dtype == "f32":
        return t
    raise ValueError(kv_dtype)


class Stream:
    """A seeded source of K/V/Q samples for one workload and seed.

    ``outliers`` is drawn once (first draw); then every call draws in the
    order the caller makes them, so callers fix the order K, V, Q.
    """

    def __init__(self, w: Workload, seed: Optional[int] = None):
        self.w = w
        self.rng = np.random.default_rng(w.seed if seed is None else seed)
        if w.outlier_channels is not None:
            self.outliers = np.asarray(w.outlier_channels, dtype=np.int64)
        else:
            self.outliers = np.sort(self.rng.choice(w.head_dim, w.n_outliers, replace=False))

    def normal(self, shape) -> np.ndarray:
        return self.rng.standard_normal(size=shape, dtype=np.float32)

    def keys(self, shape) -> torch.Tensor:
        """K samples, last axis = head_dim, outlier channels scaled."""
        x = self.normal(shape)
        x[..., self.outliers] *= np.float32(self.w.outlier_gain)
        return _to_storage(x, self.w.kv_dtype)

    def values(self, shape) -> torch.Tensor:
        return _to_storage(self.normal(shape), self.w.kv_dtype)

    def queries(self, shape) -> torch.Tensor:
        return _to_storage(self.normal(shape), self.w.kv_dtype)


def kv_pair(s: Stream, tokens: int):
    """Draw (K, V) of shape [batch, kv_heads, tokens, head_dim], K first."""
    w = s.w
    shape = (w.batch, w.kv_heads, tokens, w.head_dim)
    k = s.keys(shape)
    v = s.values(shape)
    return k, v


def decode_query(s: Stream):
    w = s.w
    return s.queries((w.batch, w.q_heads, w.head_dim))


def block_inputs(s: Stream, tq: int):
    """Own-block K/V [batch, tq, kv_heads, D] and Q [batch, tq, q_heads, D]."""
    w = s.w
    k = s.keys((w.batch, tq, w.kv_heads, w.head_dim))
    v = s.values((w.batch, tq, w.kv_heads, w.head_dim))
    q = s.queries((w.batch, tq, w.q_heads, w.head_dim))
    return q, k, v


def small(w: Workload, **changes) -> Workload:
    """A reduced copy of a workload (same dtype/codec), for CPU-sized parity."""
    return dataclasses.replace(w, **changes)


def device_kv_pair(w: Workload, tokens: int, seed: int, device="cuda", outliers=None):
    """(K, V) of shape [batch, kv_heads, tokens, head_dim] drawn on the device.

    For benchmark-scale caches only: same distribution as ``kv_pair`` (float32
    standard normals, the workload's outlier Key channels x10, cast to the
    storage dtype) from a seeded torch generator, but not the same numbers as
    the numpy draws the parity tests share with the oracle.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if outliers is None:
        outliers = Stream(w, seed).outliers
    shape = (w.batch, w.kv_heads, tokens, w.head_dim)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k[..., torch.as_tensor(outliers, device=device)] *= w.outlier_gain
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    return k.to(dt), v.to(dt)


def device_queries(w: Workload, seed: int, device="cuda"):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    q = torch.randn((w.batch, w.q_heads, w.head_dim), generator=gen, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32)
