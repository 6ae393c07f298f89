"""Run the HIP library and the CPU oracle side by side on the same inputs.

Inputs come from ``kvq_synth`` (seeded; both sides consume the same bf16 or
fp32 values).  Expected device-buffer images are built by ``oracle.layout``
from the oracle's codes, never from the library.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import kvq_synth
import quantized_kv_cache_kvq_amd as kvq
from oracle import attention as oatt
from oracle import layout as olay
from oracle.cache import (KVQuantizationStrategies, key_scales, segment_of_tokens, stacked_codes,
                          value_scales)


def note(msg: str):
    """Name the case before a GPU step, flushed, so a crash still says what ran."""
    print(msg, flush=True)
    sys.stdout.flush()


def config_for(w: kvq_synth.Workload, capacity_tokens: int, scheme=kvq.KVQ_KIVI,
               decode_kernel=kvq.KVQ_KERNEL_AUTO) -> kvq.kvq_config:
    return kvq.make_config(
        batch=w.batch, kv_heads=w.kv_heads, head_dim=w.head_dim, capacity=capacity_tokens,
        code_bits=w.code_bits, qmax=w.qmax, residual=w.residual, group=w.group,
        max_segments=None if w.group else max(capacity_tokens, 1),
        kv_dtype=kvq.KVQ_BF16 if w.kv_dtype == "bf16" else kvq.KVQ_F32,
        scheme=scheme, decode_kernel=decode_kernel)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


class Pair:
    """A device cache and the oracle state, advanced together."""

    def __init__(self, w: kvq_synth.Workload, capacity_tokens: int, scheme=kvq.KVQ_KIVI,
                 decode_kernel=kvq.KVQ_KERNEL_AUTO):
        self.w = w
        self.cfg = config_for(w, capacity_tokens, scheme, decode_kernel)
        self.cache = kvq.KVCache(self.cfg)
        self.oracle = KVQuantizationStrategies(qmax=w.qmax, eps=1e-8, scale_storage="fp16",
                                               group=w.group,
                                               axis_group=64 if scheme == kvq.KVQ_SAME_AXIS else 0)
        self.ost = None

    def append(self, k: torch.Tensor, v: torch.Tensor):
        """k, v: CPU tensors [B, H, n, D] in the workload's storage dtype."""
        self.cache.append(k.cuda(), v.cuda())
        self.ost = self.oracle.append_and_partition(self.ost, f32(k), f32(v), self.w.residual)

    # -- bit-exact comparisons ------------------------------------------------------
    def check_state(self):
        s = self.cache.state
        o = self.ost
        assert (s.quantized, s.tail, s.total, s.flushed_last, s.segments) == (
            o["quantized_tokens"], o["key_residual"].shape[-2], o["total_tokens"],
            o["flushed_tokens"], len(o["key_q_segments"]))

    def check_buffers(self):
        torch.cuda.synchronize()
        w, c, o = self.w, self.cache, self.ost
        nq, nt = c.state.quantized, c.state.tail
        cap = self.cfg.capacity
        exp_k = olay.pack_cache(stacked_codes(o, "key"), w.code_bits, cap, "key")
        exp_v = olay.pack_cache(stacked_codes(o, "value"), w.code_bits, cap, "value")
        got_k = c.k_codes.cpu().numpy()
        got_v = c.v_codes.cpu().numpy()
        assert np.array_equal(got_k, exp_k), _first_diff(got_k, exp_k)
        assert np.array_equal(got_v, exp_v), _first_diff(got_v, exp_v)
        # KIVI: one Key-scale row per segment; same-axis: per token and run
        nseg = nq if self.cfg.scheme == kvq.KVQ_SAME_AXIS else c.state.segments
        got_ks = c.k_scale[:, :, :nseg].cpu().numpy().view(np.uint16)
        exp_ks = key_scales(o).astype(np.float16).view(np.uint16)
        assert np.array_equal(got_ks, exp_ks), _first_diff(got_ks, exp_ks)
        got_vs = c.v_scale[:, :, :nq].cpu().numpy().view(np.uint16)
        exp_vs = value_scales(o).astype(np.float16).view(np.uint16)
        assert np.array_equal(got_vs, exp_vs), _first_diff(got_vs, exp_vs)
        slots = olay.ring_positions(nq, nt, c.sizes.ring)
        assert np.array_equal(f32(c.k_tail[:, :, slots]), o["key_residual"])
        assert np.array_equal(f32(c.v_tail[:, :, slots]), o["value_residual"])
        if self.cfg.group == 0:
            assert np.array_equal(c.seg_index[:nq].cpu().numpy(), segment_of_tokens(o))

    # -- attention ------------------------------------------------------------------
    def decode(self, q: torch.Tensor, num_splits: int = 0, ws=None):
        hq = q.shape[1]
        ws = ws if ws is not None else self.cache.workspace(hq, 1)
        out = torch.full((q.shape[0], hq, self.w.head_dim), float("nan"), device="cuda")
        self.cache.decode_attn(q.cuda(), out, ws, num_splits=num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ws

    def step(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, num_splits: int = 0, ws=None):
        """One kvq_decode_step (append k, v [B, H, n, D], then attend with q); the
        oracle state is advanced with the same append."""
        hq = q.shape[1]
        ws = ws if ws is not None else self.cache.workspace(hq, 1)
        out = torch.full((q.shape[0], hq, self.w.head_dim), float("nan"), device="cuda")
        self.cache.decode_step(k.cuda(), v.cuda(), q.cuda(), out, ws, num_splits=num_splits)
        torch.cuda.synchronize()
        self.ost = self.oracle.append_and_partition(self.ost, f32(k), f32(v), self.w.residual)
        return out.cpu().numpy(), ws

    def decode_ref(self, q: torch.Tensor, units=None):
        return oatt.decode_attention(self.ost, f32(q), 1.0 / math.sqrt(self.w.head_dim), units=units)

    def block(self, q: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor, num_splits: int = 0,
              ws=None, frame_tokens: int = 1):
        """q [B, tq, Hq, D], k_blk / v_blk [B, tq, Hkv, D] (CPU) -> output [B, tq, Hq, D]."""
        B, tq, hq, D = q.shape
        ws = ws if ws is not None else self.cache.workspace(hq, tq)
        out = torch.full((B, tq, hq, D), float("nan"), device="cuda")
        self.cache.block_attn(q.cuda(), k_blk.cuda(), v_blk.cuda(), out, ws, num_splits=num_splits,
                              frame_tokens=frame_tokens)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def block_ref(self, q, k_blk, v_blk, rows=None, heads=None, frame_tokens: int = 1):
        return oatt.block_attention(self.ost, f32(q), f32(k_blk), f32(v_blk),
                                    1.0 / math.sqrt(self.w.head_dim), rows=rows, heads=heads,
                                    frame_tokens=frame_tokens)


def _first_diff(a, b):
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return "equal"
    i = tuple(idx[0])
    return f"{len(idx)} mismatches; first at {i}: got {a[i]!r} expected {b[i]!r}"


def max_abs(a, b):
    m = ~np.isnan(b)
    return float(np.max(np.abs(a[m] - b[m]))) if m.any() else 0.0
