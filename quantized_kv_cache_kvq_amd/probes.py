"""Binding of libkvq_probe (``include/kvq_probe.h``): the measurement kernels
that calibrate rooflines on the machine (HBM read stream, matrix-core loop,
empty launch).  Argument marshalling only; the kernels run on the device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_probe.so")
EXPORTED = ("kvq_probe_stream_read", "kvq_probe_mfma", "kvq_probe_empty")

# flops (or integer ops) of one matrix instruction of each kind
MFMA_KINDS = {0: ("v_mfma_f32_16x16x32_bf16", 16384), 1: ("v_mfma_f32_16x16x32_f16", 16384),
              2: ("v_mfma_i32_16x16x64_i8", 32768), 3: ("v_mfma_f32_32x32x16_bf16", 32768),
              4: ("v_mfma_f32_32x32x16_f16", 32768)}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"{PROBE_LIB_PATH} is not built; run __graft_entry__.build()")
    import torch  # noqa: F401  (bind to torch's HIP runtime; see quantized_kv_cache_kvq_amd.load)
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kvq_probe_stream_read.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.kvq_probe_mfma.argtypes = [i32, i32, i32, vp, vp]
    lib.kvq_probe_empty.argtypes = [i32, vp]
    for name in EXPORTED:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream) -> int:
    import torch
    return (stream or torch.cuda.current_stream()).cuda_stream


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def stream_read(buf, workgroups: int, depth: int, sink, stream=None):
    """Read every byte of the device tensor ``buf`` once (sink: int32 device
    tensor of at least ``workgroups`` elements)."""
    _check(load().kvq_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), workgroups, depth,
                                        sink.data_ptr(), _stream(stream)), "kvq_probe_stream_read")


def mfma(kind: int, workgroups: int, iters: int, sink, stream=None):
    _check(load().kvq_probe_mfma(kind, workgroups, iters, sink.data_ptr(), _stream(stream)), "kvq_probe_mfma")


def empty(workgroups: int, stream=None):
    _check(load().kvq_probe_empty(workgroups, _stream(stream)), "kvq_probe_empty")
