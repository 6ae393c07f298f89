"""Python binding of libkvq (KIVI-style quantized KV cache on MI355X).

Argument marshalling only: every step of append, decode attention and block
attention runs in the HIP kernels of ``libkvq.so`` behind the C ABI declared
in ``include/kvq.h``.  The functions below carry the C names and take torch
tensors for device buffers (PyTorch supplies device memory and streams).
``KVCache`` owns the buffers of one uniform cache, ``PagedKVCache`` a page
pool, a caller-filled block table and one state per sequence; both check
every tensor's device, contiguity, shape and dtype before a call.  There is
no CPU fallback: if the library is not built, or no GPU is present, the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_ECAPACITY, KVQ_EWORKSPACE, KVQ_EDEVICE = range(5)
KVQ_BF16, KVQ_F32 = 0, 1
KVQ_KIVI, KVQ_SAME_AXIS = 0, 1            # kvq_scheme
KVQ_KERNEL_AUTO, KVQ_KERNEL_VALU = 0, 1   # kvq_decode_kernel

EXPORTED = ("kvq_buffer_sizes", "kvq_plan_append", "kvq_append", "kvq_workspace_size",
            "kvq_workspace_init", "kvq_decode_attn", "kvq_decode_step", "kvq_block_attn",
            "kvq_restore", "kvq_paged_page_bytes", "kvq_paged_append", "kvq_paged_decode_attn",
            "kvq_paged_decode_step", "kvq_paged_block_attn", "kvq_paged_restore", "kvq_status_str",
            "kvq_decode_attn_noalloc")


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "kv_heads", "head_dim", "capacity", "code_bits", "qmax", "residual", "group",
        "max_segments", "kv_dtype")] + [("eps", ctypes.c_float), ("scheme", ctypes.c_int32),
                                        ("decode_kernel", ctypes.c_int32)]


class kvq_state(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("quantized", "tail", "total", "flushed_last", "segments")]

    def as_tuple(self):
        return (self.quantized, self.tail, self.total, self.flushed_last, self.segments)


class kvq_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_codes", "v_codes", "k_scale", "v_scale", "k_tail", "v_tail", "seg_index")]


class kvq_paged_cache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("n_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("table_stride", ctypes.c_int32), ("k_tail", ctypes.c_void_p), ("v_tail", ctypes.c_void_p)]


class kvq_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "k_codes", "v_codes", "k_scale", "v_scale", "k_tail", "v_tail", "seg_index")] + \
        [("ring", ctypes.c_int32), ("row_bytes", ctypes.c_int32)]


class KVQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}")


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libkvq.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python -m quantized_kv_cache_kvq_amd.build")
    # torch carries its own copy of the HIP runtime under the same soname:
    # loading torch first makes the library bind to that one copy (a library
    # loaded first would pull in a second runtime, whose launches fail on
    # torch's memory and streams).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "kvq_buffer_sizes": [P(kvq_config), P(kvq_sizes)],
        "kvq_plan_append": [P(kvq_config), P(kvq_state), i64, P(kvq_state)],
        "kvq_append": [P(kvq_config), P(kvq_state), P(kvq_cache), vp, vp, i64, vp],
        "kvq_workspace_size": [P(kvq_config), i32, i32, P(sz)],
        "kvq_restore": [P(kvq_config), P(kvq_state), P(kvq_cache), vp, vp, i32, i64, vp],
        "kvq_paged_page_bytes": [P(kvq_config), P(sz)],
        "kvq_paged_append": [P(kvq_config), P(kvq_state), P(kvq_paged_cache), vp, vp, P(i64), vp],
        "kvq_paged_decode_attn": [P(kvq_config), P(kvq_state), P(kvq_paged_cache), vp, i32, f32, i32, vp, vp,
                                  sz, vp],
        "kvq_paged_restore": [P(kvq_config), P(kvq_state), P(kvq_paged_cache), vp, vp, i32, i64, vp],
        "kvq_paged_block_attn": [P(kvq_config), P(kvq_state), P(kvq_paged_cache), vp, vp, vp, i32, i32, i32, f32,
                                 i32, vp, vp, sz, vp],
        "kvq_paged_decode_step": [P(kvq_config), P(kvq_state), P(kvq_paged_cache), vp, vp, P(i64), vp, i32, f32,
                                  i32, vp, vp, sz, vp],
        "kvq_workspace_init": [vp, sz, vp],
        "kvq_decode_attn": [P(kvq_config), P(kvq_state), P(kvq_cache), vp, i32, f32, i32, vp, vp, sz, vp],
        "kvq_decode_attn_noalloc": [P(kvq_config), P(kvq_state), P(kvq_cache), vp, i32, f32, i32, vp, vp],
        "kvq_decode_step": [P(kvq_config), P(kvq_state), P(kvq_cache), vp, vp, i64, vp, i32, f32, i32,
                            vp, vp, sz, vp],
        "kvq_block_attn": [P(kvq_config), P(kvq_state), P(kvq_cache), vp, vp, vp, i32, i32, i32, f32,
                           i32, vp, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.kvq_status_str.argtypes = [ctypes.c_int]
    lib.kvq_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().kvq_status_str(status).decode()


def _check(status: int, what: str):
    if status != KVQ_OK:
        raise KVQError(status, what)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libkvq takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libkvq takes contiguous tensors")
    return t.data_ptr()


_raw_stream = None


def _stream(stream) -> Optional[int]:
    """HIP stream handle: the given torch stream's, else the current one's
    (through torch's raw query where it exists: no Stream object per call)."""
    global _raw_stream
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = ((lambda: raw(torch.cuda.current_device())) if raw is not None
                       else (lambda: torch.cuda.current_stream().cuda_stream))
    return _raw_stream()


def make_config(batch, kv_heads, head_dim, capacity, code_bits, qmax, residual, group,
                max_segments=None, kv_dtype=KVQ_BF16, eps=1e-8, scheme=None,
                decode_kernel=None) -> kvq_config:
    """scheme: KVQ_KIVI (default) or KVQ_SAME_AXIS; decode_kernel:
    KVQ_KERNEL_AUTO (default) or KVQ_KERNEL_VALU."""
    capacity = int(math.ceil(capacity / 64) * 64)
    if max_segments is None:
        max_segments = capacity // group if group else max(capacity, 1)
    return kvq_config(batch, kv_heads, head_dim, capacity, code_bits, qmax, residual, group,
                      max(max_segments, 1), kv_dtype, eps, KVQ_KIVI if scheme is None else scheme,
                      KVQ_KERNEL_AUTO if decode_kernel is None else decode_kernel)


# ---- the C entry points, one to one ----------------------------------------------

def kvq_buffer_sizes(cfg: kvq_config) -> kvq_sizes:
    out = kvq_sizes()
    _check(load().kvq_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)), "kvq_buffer_sizes")
    return out


def kvq_plan_append(cfg: kvq_config, st: kvq_state, n_new: int) -> kvq_state:
    nxt = kvq_state()
    _check(load().kvq_plan_append(ctypes.byref(cfg), ctypes.byref(st), n_new, ctypes.byref(nxt)),
           "kvq_plan_append")
    return nxt


def kvq_append(cfg, st, cache: kvq_cache, k_new, v_new, n_new: int, stream=None):
    _check(load().kvq_append(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(cache),
                             _ptr(k_new), _ptr(v_new), n_new, _stream(stream)), "kvq_append")


def kvq_restore(cfg, st, cache, k_out, v_out, out_dtype: int, ld: int, stream=None):
    _check(load().kvq_restore(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(cache), _ptr(k_out),
                              _ptr(v_out), out_dtype, ld, _stream(stream)), "kvq_restore")


def kvq_paged_page_bytes(cfg) -> int:
    n = ctypes.c_size_t()
    _check(load().kvq_paged_page_bytes(ctypes.byref(cfg), ctypes.byref(n)), "kvq_paged_page_bytes")
    return n.value


def kvq_paged_append(cfg, states, pcache, k_new, v_new, n_new, stream=None):
    if len(n_new) != cfg.batch or len(states) != cfg.batch:
        raise KVQError(KVQ_EINVAL, f"kvq_paged_append: need one count and one state per sequence ({cfg.batch})")
    counts = (ctypes.c_int64 * len(n_new))(*n_new)
    _check(load().kvq_paged_append(ctypes.byref(cfg), states, ctypes.byref(pcache), _ptr(k_new), _ptr(v_new),
                                   counts, _stream(stream)), "kvq_paged_append")


def kvq_paged_decode_attn(cfg, states, pcache, q, q_heads, softmax_scale, num_splits, out, ws, stream=None):
    _check(load().kvq_paged_decode_attn(ctypes.byref(cfg), states, ctypes.byref(pcache), _ptr(q), q_heads,
                                        softmax_scale, num_splits, _ptr(out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)),
           "kvq_paged_decode_attn")


def kvq_paged_restore(cfg, states, pcache, k_out, v_out, out_dtype: int, ld: int, stream=None):
    if len(states) != cfg.batch:
        raise KVQError(KVQ_EINVAL, f"kvq_paged_restore: need one state per sequence ({cfg.batch})")
    _check(load().kvq_paged_restore(ctypes.byref(cfg), states, ctypes.byref(pcache), _ptr(k_out), _ptr(v_out),
                                    out_dtype, ld, _stream(stream)), "kvq_paged_restore")


def kvq_paged_block_attn(cfg, states, pcache, q, k_blk, v_blk, tq, q_heads, frame_tokens, softmax_scale,
                         num_splits, out, ws, stream=None):
    if len(states) != cfg.batch:
        raise KVQError(KVQ_EINVAL, f"kvq_paged_block_attn: need one state per sequence ({cfg.batch})")
    _check(load().kvq_paged_block_attn(ctypes.byref(cfg), states, ctypes.byref(pcache), _ptr(q), _ptr(k_blk),
                                       _ptr(v_blk), tq, q_heads, frame_tokens, softmax_scale, num_splits,
                                       _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "kvq_paged_block_attn")


def kvq_paged_decode_step(cfg, states, pcache, k_new, v_new, n_new, q, q_heads, softmax_scale, num_splits, out,
                          ws, stream=None):
    if len(n_new) != cfg.batch or len(states) != cfg.batch:
        raise KVQError(KVQ_EINVAL, f"kvq_paged_decode_step: need one count and one state per sequence ({cfg.batch})")
    counts = (ctypes.c_int64 * len(n_new))(*n_new)
    _check(load().kvq_paged_decode_step(ctypes.byref(cfg), states, ctypes.byref(pcache), _ptr(k_new), _ptr(v_new),
                                        counts, _ptr(q), q_heads, softmax_scale, num_splits, _ptr(out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)), "kvq_paged_decode_step")


def kvq_workspace_size(cfg, q_heads: int, tq: int) -> int:
    n = ctypes.c_size_t()
    _check(load().kvq_workspace_size(ctypes.byref(cfg), q_heads, tq, ctypes.byref(n)),
           "kvq_workspace_size")
    return n.value


def kvq_workspace_init(ws, stream=None):
    _check(load().kvq_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "kvq_workspace_init")


def kvq_decode_attn(cfg, st, cache, q, q_heads, softmax_scale, num_splits, out, ws, stream=None):
    _check(load().kvq_decode_attn(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(cache), _ptr(q),
                                  q_heads, softmax_scale, num_splits, _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "kvq_decode_attn")


def kvq_decode_attn_noalloc(cfg, st, cache, q, q_heads, softmax_scale, num_splits, out, stream=None):
    _check(load().kvq_decode_attn_noalloc(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(cache), _ptr(q),
                                          q_heads, softmax_scale, num_splits, _ptr(out), _stream(stream)),
           "kvq_decode_attn_noalloc")


def kvq_decode_step(cfg, st, cache, k_new, v_new, n_new, q, q_heads, softmax_scale, num_splits, out, ws,
                    stream=None):
    _check(load().kvq_decode_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(cache), _ptr(k_new),
                                  _ptr(v_new), n_new, _ptr(q), q_heads, softmax_scale, num_splits,
                                  _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "kvq_decode_step")


def kvq_block_attn(cfg, st, cache, q, k_blk, v_blk, tq, q_heads, frame_tokens, softmax_scale,
                   num_splits, out, ws, stream=None):
    _check(load().kvq_block_attn(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(cache), _ptr(q),
                                 _ptr(k_blk), _ptr(v_blk), tq, q_heads, frame_tokens, softmax_scale,
                                 num_splits, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "kvq_block_attn")


# ---- device buffers (plumbing) -----------------------------------------------------

def _need(t, shape, dtypes, what: str):
    """Check a tensor handed to the library: on the device, contiguous, of the
    given shape (None = any extent) and dtype.  The C ABI takes bare pointers
    and trusts these sizes, so a mismatch here is an error, not a guess.  The
    common case is one comparison chain: these checks sit in the decode loop."""
    try:
        if t.is_cuda and t.dtype in dtypes and t.shape == shape and t.is_contiguous():
            return
    except (AttributeError, TypeError):
        pass
    bad = None
    if not getattr(t, "is_cuda", False):
        bad = "a device tensor"
    elif not t.is_contiguous():
        bad = "contiguous"
    elif t.dim() != len(shape) or any(e is not None and e != n for e, n in zip(shape, t.shape)):
        bad = f"of shape {tuple('*' if e is None else e for e in shape)}, got {tuple(t.shape)}"
    elif t.dtype not in dtypes:
        bad = f"of dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}"
    if bad:
        raise KVQError(KVQ_EINVAL, f"{what} must be {bad}")


def _check_ws(ws, i32):
    _need(ws, (ws.numel(),), i32, "workspace")


class KVCache:
    """Caller-side owner of one cache's device buffers and host state."""

    def __init__(self, cfg: kvq_config, device="cuda", zero=True):
        import torch
        self.cfg = cfg
        self.sizes = kvq_buffer_sizes(cfg)
        alloc = torch.zeros if zero else torch.empty
        B, H, D = cfg.batch, cfg.kv_heads, cfg.head_dim
        u8 = torch.uint8
        self.k_codes = alloc(B, H, self.sizes.k_codes // (B * H), dtype=u8, device=device)
        self.v_codes = alloc(B, H, self.sizes.v_codes // (B * H), dtype=u8, device=device)
        if cfg.scheme == KVQ_SAME_AXIS:     # one scale per token and run of 64 channels, K and V
            self.k_scale = alloc(B, H, cfg.capacity, D // 64, dtype=torch.float16, device=device)
            self.v_scale = alloc(B, H, cfg.capacity, D // 64, dtype=torch.float16, device=device)
        else:
            self.k_scale = alloc(B, H, cfg.max_segments, D, dtype=torch.float16, device=device)
            self.v_scale = alloc(B, H, cfg.capacity, dtype=torch.float16, device=device)
        tdt = torch.bfloat16 if cfg.kv_dtype == KVQ_BF16 else torch.float32
        self._kvdt, self._f32, self._i32 = (tdt,), (torch.float32,), (torch.int32,)
        self.k_tail = alloc(B, H, self.sizes.ring, D, dtype=tdt, device=device)
        self.v_tail = alloc(B, H, self.sizes.ring, D, dtype=tdt, device=device)
        self.seg_index = (alloc(max(cfg.capacity, 1), dtype=torch.int32, device=device)
                          if cfg.group == 0 else None)
        self.state = kvq_state()
        self.c = kvq_cache(*[_ptr(t) for t in (self.k_codes, self.v_codes, self.k_scale,
                                               self.v_scale, self.k_tail, self.v_tail,
                                               self.seg_index)])

    def _kv(self, k_new, v_new, what):
        cfg = self.cfg
        shape = (cfg.batch, cfg.kv_heads, k_new.shape[2] if k_new.dim() == 4 else None, cfg.head_dim)
        _need(k_new, shape, self._kvdt, what + " keys")
        _need(v_new, shape, self._kvdt, what + " values")

    def _q_out(self, q, out, ws, what):
        cfg = self.cfg
        shape = (cfg.batch, q.shape[1] if q.dim() == 3 else None, cfg.head_dim)
        _need(q, shape, self._kvdt, what + " queries")
        _need(out, shape, self._f32, what + " output")
        _check_ws(ws, self._i32)

    def append(self, k_new, v_new, stream=None):
        self._kv(k_new, v_new, "append")
        kvq_append(self.cfg, self.state, self.c, k_new, v_new, k_new.shape[2], stream)

    def restore(self, k_out, v_out, stream=None):
        """Restored quantized prefix into k_out / v_out [B, Hkv, ld, D] (fp32 or bf16)."""
        import torch
        B, H, D = self.cfg.batch, self.cfg.kv_heads, self.cfg.head_dim
        shape = (B, H, k_out.shape[2] if k_out.dim() == 4 else None, D)
        _need(k_out, shape, (torch.float32, torch.bfloat16), "restore keys")
        _need(v_out, shape, (k_out.dtype,), "restore values")
        dt = KVQ_BF16 if k_out.dtype == torch.bfloat16 else KVQ_F32
        kvq_restore(self.cfg, self.state, self.c, k_out, v_out, dt, k_out.shape[2], stream)

    def workspace(self, q_heads: int, tq: int = 1, stream=None):
        import torch
        n = kvq_workspace_size(self.cfg, q_heads, tq)
        ws = torch.empty(n // 4, dtype=torch.int32, device=self.k_codes.device)
        kvq_workspace_init(ws, stream)
        return ws

    def decode_attn(self, q, out, ws, softmax_scale=None, num_splits=0, stream=None):
        D = self.cfg.head_dim
        s = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
        self._q_out(q, out, ws, "decode")
        kvq_decode_attn(self.cfg, self.state, self.c, q, q.shape[1], s, num_splits, out, ws, stream)

    def decode_step(self, k_new, v_new, q, out, ws, softmax_scale=None, num_splits=0, stream=None):
        """Append k_new/v_new [B, Hkv, n, D], then attend with q (one call)."""
        D = self.cfg.head_dim
        s = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
        self._kv(k_new, v_new, "decode step")
        self._q_out(q, out, ws, "decode step")
        kvq_decode_step(self.cfg, self.state, self.c, k_new, v_new, k_new.shape[2], q, q.shape[1], s,
                        num_splits, out, ws, stream)

    def block_attn(self, q, k_blk, v_blk, out, ws, softmax_scale=None, num_splits=0, stream=None,
                   frame_tokens=1):
        """frame_tokens = F: bidirectional inside frames of F positions, causal
        across frames; 1 = token-causal."""
        D = self.cfg.head_dim
        s = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
        B, H = self.cfg.batch, self.cfg.kv_heads
        ok4 = q.dim() == 4
        qshape = (B, q.shape[1] if ok4 else None, q.shape[2] if ok4 else None, D)
        kshape = (B, qshape[1], H, D)
        _need(q, qshape, self._kvdt, "block queries")
        _need(k_blk, kshape, self._kvdt, "block keys")
        _need(v_blk, kshape, self._kvdt, "block values")
        _need(out, qshape, self._f32, "block output")
        _check_ws(ws, self._i32)
        kvq_block_attn(self.cfg, self.state, self.c, q, k_blk, v_blk, q.shape[1], q.shape[2],
                       frame_tokens, s, num_splits, out, ws, stream)


class PagedKVCache:
    """Caller-side owner of a paged cache: the page pool, the block table
    (int32 [batch, table_stride], device, filled by the caller) and the dense
    windows, plus one kvq_state per sequence."""

    def __init__(self, cfg: kvq_config, n_pages: int, block_table, device="cuda"):
        import torch
        self.cfg = cfg
        _need(block_table, (cfg.batch, block_table.shape[-1] if block_table.dim() == 2 else None),
              (torch.int32,), "block table")
        self.page_bytes = kvq_paged_page_bytes(cfg)
        self.pool = torch.zeros(n_pages * self.page_bytes, dtype=torch.uint8, device=device)
        self.table = block_table
        sizes = kvq_buffer_sizes(cfg)
        tdt = torch.bfloat16 if cfg.kv_dtype == KVQ_BF16 else torch.float32
        self._kvdt, self._f32, self._i32 = (tdt,), (torch.float32,), (torch.int32,)
        B, H, D = cfg.batch, cfg.kv_heads, cfg.head_dim
        self.k_tail = torch.zeros(B, H, sizes.ring, D, dtype=tdt, device=device)
        self.v_tail = torch.zeros(B, H, sizes.ring, D, dtype=tdt, device=device)
        self.ring = sizes.ring
        self.states = (kvq_state * B)()
        self.c = kvq_paged_cache(_ptr(self.pool), n_pages, _ptr(block_table), block_table.shape[1],
                                 _ptr(self.k_tail), _ptr(self.v_tail))

    def append(self, k_new, v_new, n_new, stream=None):
        """k_new, v_new [B, Hkv, max_n, D]; sequence b appends its first n_new[b] rows."""
        cfg = self.cfg
        n_new = list(n_new)
        shape = (cfg.batch, cfg.kv_heads, k_new.shape[2] if k_new.dim() == 4 else None, cfg.head_dim)
        _need(k_new, shape, self._kvdt, "paged append keys")
        _need(v_new, shape, self._kvdt, "paged append values")
        if not n_new or max(n_new) != k_new.shape[2]:
            # the library reads sequence b's rows at a stride of max(n_new) rows
            raise KVQError(KVQ_EINVAL, f"paged append: k_new / v_new must hold max(n_new) rows, "
                                       f"got {k_new.shape[2]} rows for counts {n_new}")
        kvq_paged_append(self.cfg, self.states, self.c, k_new, v_new, list(n_new), stream)

    def workspace(self, q_heads: int, tq: int = 1, stream=None):
        import torch
        n = kvq_workspace_size(self.cfg, q_heads, tq)
        ws = torch.empty(n // 4, dtype=torch.int32, device=self.pool.device)
        kvq_workspace_init(ws, stream)
        return ws

    def decode_attn(self, q, out, ws, softmax_scale=None, num_splits=0, stream=None):
        D = self.cfg.head_dim
        s = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
        shape = (self.cfg.batch, q.shape[1] if q.dim() == 3 else None, D)
        _need(q, shape, self._kvdt, "paged decode queries")
        _need(out, shape, self._f32, "paged decode output")
        _check_ws(ws, self._i32)
        kvq_paged_decode_attn(self.cfg, self.states, self.c, q, q.shape[1], s, num_splits, out, ws, stream)

    def restore(self, k_out, v_out, stream=None):
        """Every sequence's restored prefix into k_out / v_out [B, Hkv, ld, D] (fp32 or bf16)."""
        import torch
        cfg = self.cfg
        shape = (cfg.batch, cfg.kv_heads, k_out.shape[2] if k_out.dim() == 4 else None, cfg.head_dim)
        _need(k_out, shape, (torch.float32, torch.bfloat16), "paged restore keys")
        _need(v_out, shape, (k_out.dtype,), "paged restore values")
        dt = KVQ_BF16 if k_out.dtype == torch.bfloat16 else KVQ_F32
        kvq_paged_restore(cfg, self.states, self.c, k_out, v_out, dt, k_out.shape[2], stream)

    def block_attn(self, q, k_blk, v_blk, out, ws, softmax_scale=None, num_splits=0, stream=None,
                   frame_tokens=1):
        """q [B, tq, Hq, D], k_blk / v_blk [B, tq, Hkv, D]: each sequence's block of tq
        queries after its own cached tokens (frame mask as for KVCache.block_attn)."""
        cfg = self.cfg
        D, B, H = cfg.head_dim, cfg.batch, cfg.kv_heads
        ok4 = q.dim() == 4
        qshape = (B, q.shape[1] if ok4 else None, q.shape[2] if ok4 else None, D)
        kshape = (B, qshape[1], H, D)
        _need(q, qshape, self._kvdt, "paged block queries")
        _need(k_blk, kshape, self._kvdt, "paged block keys")
        _need(v_blk, kshape, self._kvdt, "paged block values")
        _need(out, qshape, self._f32, "paged block output")
        _check_ws(ws, self._i32)
        s = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
        kvq_paged_block_attn(cfg, self.states, self.c, q, k_blk, v_blk, q.shape[1], q.shape[2], frame_tokens, s,
                             num_splits, out, ws, stream)

    def decode_step(self, k_new, v_new, n_new, q, out, ws, softmax_scale=None, num_splits=0, stream=None):
        """Append sequence b's first n_new[b] rows of k_new / v_new [B, Hkv, max_n, D],
        then attend with q [B, Hq, D] over every cache (one call)."""
        cfg = self.cfg
        D = cfg.head_dim
        n_new = list(n_new)
        shape = (cfg.batch, cfg.kv_heads, k_new.shape[2] if k_new.dim() == 4 else None, D)
        _need(k_new, shape, self._kvdt, "paged step keys")
        _need(v_new, shape, self._kvdt, "paged step values")
        if not n_new or max(n_new) != k_new.shape[2]:
            # the library reads sequence b's rows at a stride of max(n_new) rows
            raise KVQError(KVQ_EINVAL, f"paged step: k_new / v_new must hold max(n_new) rows, "
                                       f"got {k_new.shape[2]} rows for counts {n_new}")
        qshape = (cfg.batch, q.shape[1] if q.dim() == 3 else None, D)
        _need(q, qshape, self._kvdt, "paged step queries")
        _need(out, qshape, self._f32, "paged step output")
        _check_ws(ws, self._i32)
        s = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
        kvq_paged_decode_step(cfg, self.states, self.c, k_new, v_new, n_new, q, q.shape[1], s, num_splits, out, ws,
                              stream)
