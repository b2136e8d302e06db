"""Thin Python binding of libkvq.so (include/kvq.h).

The functions below carry the C entry points' names and only marshal
arguments: every step of the decode path runs in the library's HIP kernels.
PyTorch supplies device memory and the stream.  If the library is not built
the import of any entry point fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

HEAD_DIM = 128
K_GROUP = 32
COL_WARMUP = 64
RING_WINDOW = 128
MAX_KV_HEADS = 64
MAX_CAPACITY = 1 << 24
ALL_SEQS = -1

OK, EINVAL, ECAPACITY, ESTATE, EDEVICE = 0, -1, -2, -3, -4
KIND_F32, KIND_Q8, KIND_I8 = 1, 2, 3
BUF_K, BUF_V, BUF_KQ, BUF_KS, BUF_VQ, BUF_VS, BUF_KCOL, BUF_VCOL = range(8)

_P = ctypes.c_void_p


class kvq_cache(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32), ("n_live", ctypes.c_int32),
        ("live_slot", ctypes.c_int8 * MAX_KV_HEADS),
        ("len", _P), ("frozen", _P),
        ("k", _P), ("v", _P), ("kq", _P), ("ks", _P), ("vq", _P), ("vs", _P),
        ("kcol", _P), ("vcol", _P),
    ]


class kvq_ring(ctypes.Structure):
    _fields_ = [("prefill_len", ctypes.c_int32), ("ring_len", ctypes.c_int32),
                ("ring_pos", ctypes.c_int32), ("epoch", ctypes.c_int32),
                ("writes", ctypes.c_int64)]


class kvq_ring_checkpoint(ctypes.Structure):
    _fields_ = [("cache", _P), ("seq", ctypes.c_int32), ("prefill_len", ctypes.c_int32),
                ("ring_len", ctypes.c_int32), ("ring_pos", ctypes.c_int32), ("epoch", ctypes.c_int32),
                ("stream", ctypes.c_int32), ("writes", ctypes.c_int64)]


class kvq_decode_opts(ctypes.Structure):
    _fields_ = [("first", _P), ("softcap", ctypes.c_float), ("reserved", ctypes.c_int32), ("sinks", _P)]


_lib = None

# (name, restype, argtypes) of every exported entry point
_SIGNATURES = [
    ("kvq_cache_init", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _P, _P, _P]),
    ("kvq_buffer_bytes", ctypes.c_size_t, [_P, ctypes.c_int]),
    ("kvq_cache_bytes", ctypes.c_size_t, [_P]),
    ("kv_append_f32", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, _P, _P, _P]),
    ("kv_append_q8", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, _P, _P, _P]),
    ("kv_freeze_col_and_requant", ctypes.c_int, [_P, ctypes.c_int, _P]),
    ("kv_append_i8", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int, _P, _P, _P]),
    ("decode_attn_i8", ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P]),
    ("kvq_workspace_bytes", ctypes.c_size_t, [_P, ctypes.c_int]),
    ("decode_attn_f32", ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P]),
    ("decode_attn_q8", ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P]),
    ("decode_attn_f32_ex", ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("decode_attn_q8_ex", ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("rswa_record_prefill", ctypes.c_int, [_P, _P, ctypes.c_int]),
    ("rswa_decode", ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("rswa_checkpoint", ctypes.c_int, [_P, _P, ctypes.c_int, _P]),
    ("rswa_rollback_to", ctypes.c_int, [_P, _P, ctypes.c_int, _P]),
    ("kv_truncate_last", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int]),
    ("kv_trim_window", ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int64, _P, _P]),
    ("rswa_verify", ctypes.c_int, [_P, _P, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("kvq_verify_workspace_bytes", ctypes.c_size_t, [_P, ctypes.c_int, ctypes.c_int]),
    ("rswa_shared_record_prefill", ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int]),
    ("rswa_shared_decode", ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    ("decode_attn_q8_noalloc", ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P]),
    ("rswa_shared_checkpoint", ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, _P]),
    ("rswa_shared_rollback_to", ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, _P]),
    ("kvq_last_error", ctypes.c_char_p, []),
]


def lib():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built (%s); run `python -m int8_kv_cache_decode_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class KvqError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("kvq error %d: %s" % (code, message))
        self.code = code
        self.message = message


def last_error() -> str:
    return lib().kvq_last_error().decode()


def _check(rc: int) -> None:
    if rc != OK:
        raise KvqError(rc, last_error())


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Cache object: the kvq_cache struct, its host counters and (optionally) its
# device buffers allocated through torch.
# ---------------------------------------------------------------------------
class KvCache:
    def __init__(self, kind: int, batch: int, n_kv_heads: int, capacity: int, alive=None,
                 device: str = "cuda", allocate: bool = True):
        self.c = kvq_cache()
        self.len = np.zeros(batch, np.int32)
        self.frozen = np.zeros(batch, np.uint8)
        self._alive = None if alive is None else np.ascontiguousarray(alive, np.uint8)
        rc = lib().kvq_cache_init(ctypes.byref(self.c), kind, batch, n_kv_heads, HEAD_DIM, capacity,
                                  None if self._alive is None else self._alive.ctypes.data,
                                  self.len.ctypes.data, self.frozen.ctypes.data)
        _check(rc)
        self.kind, self.batch, self.n_kv_heads, self.capacity = kind, batch, n_kv_heads, capacity
        self.n_live = self.c.n_live
        self.buffers = {}
        self._ws = None
        if allocate:
            import torch
            names = {KIND_F32: ("k", "v"), KIND_Q8: ("kq", "ks", "vq", "vs", "kcol", "vcol"),
                     KIND_I8: ("kq", "ks", "vq", "vs")}[kind]
            ids = {"k": BUF_K, "v": BUF_V, "kq": BUF_KQ, "ks": BUF_KS, "vq": BUF_VQ, "vs": BUF_VS,
                   "kcol": BUF_KCOL, "vcol": BUF_VCOL}
            for n in names:
                nbytes = lib().kvq_buffer_bytes(ctypes.byref(self.c), ids[n])
                t = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
                self.buffers[n] = t
                setattr(self.c, n, t.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.c)

    # typed views of the device storage
    def view(self, name: str):
        import torch
        B, H, C = self.batch, self.n_live, self.capacity
        t = self.buffers[name]
        if name in ("k", "v"):
            return t[: B * H * C * HEAD_DIM * 4].view(torch.float32).view(B, H, C, HEAD_DIM)
        if name == "kq":
            # K codes are stored tile-major (16-row tiles in MFMA operand
            # order); this returns them row-major, as a copy
            C16 = (C + 15) // 16 * 16
            raw = t[: B * H * C16 * HEAD_DIM].view(torch.int8).view(B, H, C16 // 16, 2, 4, 16, 16)
            return raw.permute(0, 1, 2, 5, 3, 4, 6).reshape(B, H, C16, HEAD_DIM)[:, :, :C]
        if name == "vq":
            return t[: B * H * C * HEAD_DIM].view(torch.int8).view(B, H, C, HEAD_DIM)
        if name == "ks" and self.kind == KIND_I8:
            return t[: B * H * C * 4].view(torch.float32).view(B, H, C)
        if name == "ks":
            return t[: B * H * C * 16].view(torch.float32).view(B, H, C, 4)
        if name == "vs":
            return t[: B * H * C * 4].view(torch.float32).view(B, H, C)
        return t[: B * H * HEAD_DIM * 4].view(torch.float32).view(B, H, HEAD_DIM)

    def workspace(self, n_q_heads: int):
        import torch
        need = kvq_workspace_bytes(self, n_q_heads)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.buffers[next(iter(self.buffers))].device)
        return self._ws

    def cache_bytes(self) -> int:
        return kvq_cache_bytes(self)


class Rings:
    """Host array of kvq_ring, one per sequence of an R-SWA cache."""

    def __init__(self, batch: int):
        self.arr = (kvq_ring * batch)()
        for r in self.arr:
            r.prefill_len = -1

    @property
    def ref(self):
        return ctypes.byref(self.arr)

    def __getitem__(self, i) -> kvq_ring:
        return self.arr[i]


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def kvq_buffer_bytes(cache: KvCache, which: int) -> int:
    return lib().kvq_buffer_bytes(cache.ref, which)


def kvq_cache_bytes(cache: KvCache) -> int:
    return lib().kvq_cache_bytes(cache.ref)


def kvq_workspace_bytes(cache: KvCache, n_q_heads: int) -> int:
    return lib().kvq_workspace_bytes(cache.ref, n_q_heads)


def kv_append_f32(cache: KvCache, seq: int, n_rows: int, k_new, v_new, stream=None) -> None:
    _check(lib().kv_append_f32(cache.ref, seq, n_rows, _ptr(k_new), _ptr(v_new), _stream(stream)))


def kv_append_q8(cache: KvCache, seq: int, n_rows: int, k_new, v_new, stream=None) -> None:
    _check(lib().kv_append_q8(cache.ref, seq, n_rows, _ptr(k_new), _ptr(v_new), _stream(stream)))


def kv_append_i8(cache: KvCache, seq: int, n_rows: int, k_new, v_new, stream=None) -> None:
    _check(lib().kv_append_i8(cache.ref, seq, n_rows, _ptr(k_new), _ptr(v_new), _stream(stream)))


def decode_attn_i8(cache: KvCache, n_q_heads: int, q, out, ws=None, ws_bytes=None, stream=None) -> None:
    ws = cache.workspace(n_q_heads) if ws is None else ws
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().decode_attn_i8(cache.ref, n_q_heads, _ptr(q), _ptr(out), _ptr(ws), nb, _stream(stream)))


def kv_freeze_col_and_requant(cache: KvCache, seq: int, stream=None) -> None:
    _check(lib().kv_freeze_col_and_requant(cache.ref, seq, _stream(stream)))


def decode_attn_f32(cache: KvCache, n_q_heads: int, q, out, ws=None, ws_bytes=None, stream=None) -> None:
    ws = cache.workspace(n_q_heads) if ws is None else ws
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().decode_attn_f32(cache.ref, n_q_heads, _ptr(q), _ptr(out), _ptr(ws), nb, _stream(stream)))


def decode_attn_q8(cache: KvCache, n_q_heads: int, q, out, ws=None, ws_bytes=None, stream=None) -> None:
    ws = cache.workspace(n_q_heads) if ws is None else ws
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().decode_attn_q8(cache.ref, n_q_heads, _ptr(q), _ptr(out), _ptr(ws), nb, _stream(stream)))


class DecodeOpts:
    """kvq_decode_opts: first (host int32 [batch] or None), softcap (0 = off),
    sinks (device float [n_q_heads] tensor or None).  Keeps the host array
    alive for the call."""

    def __init__(self, first=None, softcap: float = 0.0, sinks=None):
        self.first = None if first is None else np.ascontiguousarray(first, np.int32)
        self.sinks = sinks
        self.c = kvq_decode_opts()
        self.c.first = None if self.first is None else self.first.ctypes.data
        self.c.softcap = float(softcap)
        self.c.reserved = 0
        self.c.sinks = _ptr(sinks)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def decode_attn_f32_ex(cache: KvCache, n_q_heads: int, q, out, opts: Optional[DecodeOpts] = None,
                       ws=None, ws_bytes=None, stream=None) -> None:
    ws = cache.workspace(n_q_heads) if ws is None else ws
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().decode_attn_f32_ex(cache.ref, n_q_heads, _ptr(q), _ptr(out), None if opts is None else opts.ref,
                                    _ptr(ws), nb, _stream(stream)))


def decode_attn_q8_ex(cache: KvCache, n_q_heads: int, q, out, opts: Optional[DecodeOpts] = None,
                      ws=None, ws_bytes=None, stream=None) -> None:
    ws = cache.workspace(n_q_heads) if ws is None else ws
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().decode_attn_q8_ex(cache.ref, n_q_heads, _ptr(q), _ptr(out), None if opts is None else opts.ref,
                                   _ptr(ws), nb, _stream(stream)))


def rswa_record_prefill(cache: KvCache, rings: Rings, seq: int) -> None:
    _check(lib().rswa_record_prefill(cache.ref, rings.ref, seq))


def rswa_decode(cache: KvCache, rings: Rings, n_q_heads: int, q, k_new, v_new, out,
                ws=None, ws_bytes=None, stream=None) -> None:
    ws = cache.workspace(n_q_heads) if ws is None else ws
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().rswa_decode(cache.ref, rings.ref, n_q_heads, _ptr(q), _ptr(k_new), _ptr(v_new),
                             _ptr(out), _ptr(ws), nb, _stream(stream)))


def rswa_checkpoint(cache: KvCache, rings: Rings, seq: int) -> kvq_ring_checkpoint:
    cp = kvq_ring_checkpoint()
    _check(lib().rswa_checkpoint(cache.ref, rings.ref, seq, ctypes.byref(cp)))
    return cp


def rswa_rollback_to(cache: KvCache, rings: Rings, seq: int, cp: kvq_ring_checkpoint) -> None:
    _check(lib().rswa_rollback_to(cache.ref, rings.ref, seq, ctypes.byref(cp)))


def kv_truncate_last(cache: KvCache, seq: int, n_drop: int) -> None:
    _check(lib().kv_truncate_last(cache.ref, seq, n_drop))


def kv_trim_window(cache: KvCache, seq: int, base, w: int, slack: int, align: int, anchor: int = -1,
                   stream=None):
    """Returns (new base, rows dropped).  seq == ALL_SEQS: base is one
    position per sequence and the result is (bases, dropped) as int64 /
    int32 arrays."""
    if seq == ALL_SEQS:
        b = np.ascontiguousarray(base, np.int64).copy()
        d = np.zeros(b.shape[0], np.int32)
        if b.shape[0] != cache.batch:
            raise ValueError("one base per sequence")
        _check(lib().kv_trim_window(cache.ref, seq, b.ctypes.data, w, slack, align, anchor, d.ctypes.data,
                                    _stream(stream)))
        return b, d
    b = ctypes.c_int64(base)
    d = ctypes.c_int(0)
    _check(lib().kv_trim_window(cache.ref, seq, ctypes.byref(b), w, slack, align, anchor, ctypes.byref(d),
                                _stream(stream)))
    return b.value, d.value


def kvq_verify_workspace_bytes(cache: KvCache, n_q_heads: int, n_draft: int) -> int:
    return lib().kvq_verify_workspace_bytes(cache.ref, n_q_heads, n_draft)


def rswa_verify(cache: KvCache, rings: Rings, n_q_heads: int, n_draft: int, q, k_draft, v_draft, out,
                ws=None, ws_bytes=None, stream=None) -> None:
    if ws is None:
        import torch
        need = kvq_verify_workspace_bytes(cache, n_q_heads, n_draft)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=out.device)
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().rswa_verify(cache.ref, rings.ref, n_q_heads, n_draft, _ptr(q), _ptr(k_draft), _ptr(v_draft),
                             _ptr(out), _ptr(ws), nb, _stream(stream)))


def rswa_shared_record_prefill(cache: KvCache, seq: int, rings: Rings, n_streams: int) -> None:
    _check(lib().rswa_shared_record_prefill(cache.ref, seq, rings.ref, n_streams))


def rswa_shared_decode(cache: KvCache, seq: int, rings: Rings, n_streams: int, n_q_heads: int, q, k_new, v_new,
                       out, ws=None, ws_bytes=None, stream=None) -> None:
    if ws is None:
        import torch
        need = kvq_verify_workspace_bytes(cache, n_q_heads, n_streams)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=out.device)
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().rswa_shared_decode(cache.ref, seq, rings.ref, n_streams, n_q_heads, _ptr(q), _ptr(k_new),
                                    _ptr(v_new), _ptr(out), _ptr(ws), nb, _stream(stream)))


def rswa_shared_checkpoint(cache: KvCache, seq: int, rings: Rings, n_streams: int, s: int) -> kvq_ring_checkpoint:
    cp = kvq_ring_checkpoint()
    _check(lib().rswa_shared_checkpoint(cache.ref, seq, rings.ref, n_streams, s, ctypes.byref(cp)))
    return cp


def rswa_shared_rollback_to(cache: KvCache, seq: int, rings: Rings, n_streams: int, s: int,
                            cp: kvq_ring_checkpoint) -> None:
    _check(lib().rswa_shared_rollback_to(cache.ref, seq, rings.ref, n_streams, s, ctypes.byref(cp)))


def decode_attn_q8_noalloc(cache: KvCache, n_q_heads: int, q, out, stream=None) -> None:
    _check(lib().decode_attn_q8_noalloc(cache.ref, n_q_heads, _ptr(q), _ptr(out), _stream(stream)))
