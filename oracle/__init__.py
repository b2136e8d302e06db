"""CPU oracle for int8/f32 KV-cache decode attention -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
oracle never imports the product: the two share no code.  The only module both
sides use is ``workloads`` (seeded input generators, no arithmetic of the
method).

What is here:
  * ``kvq_oracle.c`` (built into ``libkvq_oracle.so`` with gcc): attention by
    its definition in float64, and the q8_2f codec step by step in IEEE f32.
  * this file: ctypes marshalling, a per-head q8 cache state, a batch driver
    that runs independent (sequence, KV group) units on a thread pool (ctypes
    releases the GIL, the arithmetic inside one unit is untouched), and the
    R-SWA ring cursor model in plain Python.

Sources (web pages):
  [P1] cortiq-engine 0.3.4, src/cortiq_engine/kv_cache.rs
  [P3] franken_ocr 0.8.0, src/native_engine/rswa.rs
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

COL_WARMUP = 64   # [P1] const KV_COL_WARMUP
K_GROUP = 32      # [P1] const KV_K_GROUP
RING_W = 128      # [P3] const RING_WINDOW

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.orc_quant_row.argtypes = [P, P, i, i, P, P]
        L.orc_quant_row.restype = None
        L.orc_freeze_one.argtypes = [i, i, i, P, P, P]
        L.orc_freeze_one.restype = i
        L.orc_q8_append_head.argtypes = [i, i, i, P, P, i, P, P, P, P, P, P, P, P]
        L.orc_q8_append_head.restype = i
        L.orc_q8_freeze_head.argtypes = [i, P, P, P, P, P, P, i, P]
        L.orc_q8_freeze_head.restype = i
        L.orc_attend_f32.argtypes = [i, i, i, P, P, P, P]
        L.orc_attend_f32.restype = None
        L.orc_attend_q8.argtypes = [i, i, i, P, P, P, P, P, P, P, P]
        L.orc_attend_q8.restype = None
        d = ctypes.c_double
        L.orc_attend_f32_ex.argtypes = [i, i, i, P, P, P, i, d, P, P]
        L.orc_attend_f32_ex.restype = None
        L.orc_attend_q8_ex.argtypes = [i, i, i, P, P, P, P, P, P, P, i, d, P, P]
        L.orc_attend_q8_ex.restype = None
        L.orc_quant_row_i8.argtypes = [P, i, P]
        L.orc_quant_row_i8.restype = ctypes.c_float
        L.orc_quant_rows_i8.argtypes = [i, i, P, P, P]
        L.orc_quant_rows_i8.restype = None
        L.orc_attend_i8.argtypes = [i, i, i, P, P, P, P, P, P]
        L.orc_attend_i8.restype = None
        L.orc_attend_i8_ex.argtypes = [i, i, i, P, P, P, P, P, i, P, P]
        L.orc_attend_i8_ex.restype = None
        L.orc_weights_f32.argtypes = [i, i, P, P, P]
        L.orc_weights_f32.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# Codec ([P1] LayerKvCache::quant_row / freeze_cols / append)
# --------------------------------------------------------------------------
def quant_row(x, col=None, group: int = K_GROUP):
    """One row -> (int8 codes [hd], f32 scales [ceil(hd/group)])."""
    x = _f32(x)
    hd = x.shape[0]
    colv = None if col is None else _f32(col)
    q = np.zeros(hd, np.int8)
    s = np.zeros(-(-hd // group), np.float32)
    _load().orc_quant_row(_p(x), _p(colv), hd, group, _p(q), _p(s))
    return q, s


def freeze_one(codes: np.ndarray, scales: np.ndarray, group: int):
    """Freeze one head's K (group 32) or V (group hd) block in place.

    codes [n][hd] int8 and scales [n][ns] f32 are requantised in place;
    returns the column field [hd] (or None when n == 0)."""
    n, hd = codes.shape
    assert codes.flags.c_contiguous and scales.flags.c_contiguous
    col = np.zeros(hd, np.float32)
    done = _load().orc_freeze_one(n, hd, group, _p(codes), _p(scales), _p(col))
    return col if done else None


class Q8Head:
    """q8_2f storage of ONE live KV head of one sequence ([P1] LayerKvCache
    fields kq/ks/vq/vs/kcol/vcol restricted to one head)."""

    def __init__(self, cap: int, hd: int = 128):
        self.cap, self.hd = cap, hd
        ng = -(-hd // K_GROUP)
        self.kq = np.zeros((cap, hd), np.int8)
        self.ks = np.zeros((cap, ng), np.float32)
        self.vq = np.zeros((cap, hd), np.int8)
        self.vs = np.zeros(cap, np.float32)
        self.kcol = np.ones(hd, np.float32)
        self.vcol = np.ones(hd, np.float32)
        self._n = ctypes.c_int(0)
        self._frozen = ctypes.c_int(0)

    @property
    def n(self) -> int:
        return self._n.value

    @property
    def frozen(self) -> bool:
        return bool(self._frozen.value)

    def append(self, k_rows, v_rows) -> None:
        """Append rows (k_rows/v_rows: [n_new][hd]) one at a time, freezing at
        the start of the append that finds >= 64 stored rows."""
        k_rows, v_rows = _f32(k_rows), _f32(v_rows)
        n_new, hd = k_rows.shape
        assert hd == self.hd and v_rows.shape == k_rows.shape
        rc = _load().orc_q8_append_head(
            hd, self.cap, n_new, _p(k_rows), _p(v_rows), hd,
            _p(self.kq), _p(self.ks), _p(self.vq), _p(self.vs),
            _p(self.kcol), _p(self.vcol),
            ctypes.addressof(self._n), ctypes.addressof(self._frozen))
        if rc != 0:
            raise ValueError("oracle q8 append: capacity exceeded")

    def truncate_last(self, n_drop: int) -> None:
        """[P2] LayerKvCache::truncate_last on this head: the last
        min(n_drop, n) rows are dropped; the column fields stay as they are
        (a frozen field stays frozen, so later rows quantise against it)."""
        self._n.value = truncate_last(self.n, n_drop)

    def freeze(self) -> bool:
        return bool(_load().orc_q8_freeze_head(
            self.hd, _p(self.kq), _p(self.ks), _p(self.vq), _p(self.vs),
            _p(self.kcol), _p(self.vcol), self.n, ctypes.addressof(self._frozen)))

    def dequant_k(self) -> np.ndarray:
        """K^ in float64: code * group scale * column field."""
        n = self.n
        sc = np.repeat(self.ks[:n].astype(np.float64), K_GROUP, axis=1)[:, : self.hd]
        col = self.kcol.astype(np.float64) if self.frozen else 1.0
        return self.kq[:n].astype(np.float64) * sc * col

    def dequant_v(self) -> np.ndarray:
        n = self.n
        col = self.vcol.astype(np.float64) if self.frozen else 1.0
        return self.vq[:n].astype(np.float64) * self.vs[:n, None].astype(np.float64) * col


def quant_row_i8(x):
    """[P3] quantize_row_i8 of one f32 row -> (codes int8 [hd], scale f32)."""
    x = _f32(x)
    q = np.zeros(x.shape[0], np.int8)
    sc = _load().orc_quant_row_i8(_p(x), x.shape[0], _p(q))
    return q, np.float32(sc)


class I8Head:
    """Per-row int8 storage of ONE live KV head ([P3] Int8Kv: codes and one
    f32 scale per row, for K and for V)."""

    def __init__(self, cap: int, hd: int = 128):
        self.cap, self.hd, self.n = cap, hd, 0
        self.kq = np.zeros((cap, hd), np.int8)
        self.ks = np.zeros(cap, np.float32)
        self.vq = np.zeros((cap, hd), np.int8)
        self.vs = np.zeros(cap, np.float32)

    def append(self, k_rows, v_rows) -> None:
        k_rows, v_rows = _f32(k_rows), _f32(v_rows)
        n_new = k_rows.shape[0]
        if self.n + n_new > self.cap:
            raise ValueError("oracle i8 append: capacity exceeded")
        n0 = self.n
        for src, q, sc in ((k_rows, self.kq, self.ks), (v_rows, self.vq, self.vs)):
            qq = np.zeros((n_new, self.hd), np.int8)
            ss = np.zeros(n_new, np.float32)
            _load().orc_quant_rows_i8(n_new, self.hd, _p(np.ascontiguousarray(src)), _p(qq), _p(ss))
            q[n0:n0 + n_new], sc[n0:n0 + n_new] = qq, ss
        self.n += n_new

    def truncate_last(self, n_drop: int) -> None:
        """[P2] LayerKvCache::truncate_last: the last min(n_drop, n) rows are
        dropped (per-row codes do not depend on other rows)."""
        self.n = truncate_last(self.n, n_drop)

    def dequant_k(self) -> np.ndarray:
        return self.kq[: self.n].astype(np.float64) * self.ks[: self.n, None].astype(np.float64)

    def dequant_v(self) -> np.ndarray:
        return self.vq[: self.n].astype(np.float64) * self.vs[: self.n, None].astype(np.float64)


# --------------------------------------------------------------------------
# Attention by definition (float64)
# --------------------------------------------------------------------------
def _sinks(sinks, hpk):
    if sinks is None:
        return None
    z = np.ascontiguousarray(np.asarray(sinks, np.float32).reshape(-1))
    assert z.shape[0] == hpk, "one sink logit per Q head of the group"
    return z


def attend_f32(q, k, v, first: int = 0, softcap: float = 0.0, sinks=None) -> np.ndarray:
    """q [hpk][hd] (or [hd]), k/v [n][hd] f32 -> out float64 like q.

    first / softcap / sinks: [P2] attend_group_upto's visible-row start,
    Gemma-2 logit soft-cap (0 = off) and per-head learned sink logits
    (None = no sinks)."""
    q = _f32(q)
    squeeze = q.ndim == 1
    q2 = q.reshape(1, -1) if squeeze else q
    hpk, hd = q2.shape
    k, v = _f32(k).reshape(-1, hd), _f32(v).reshape(-1, hd)
    n = k.shape[0]
    out = np.zeros((hpk, hd), np.float64)
    z = _sinks(sinks, hpk)
    _load().orc_attend_f32_ex(n, hd, hpk, _p(q2), _p(k), _p(v), int(first), float(softcap), _p(z), _p(out))
    return out[0] if squeeze else out


def attend_q8(q, head: Q8Head, first: int = 0, softcap: float = 0.0, sinks=None) -> np.ndarray:
    q = _f32(q)
    squeeze = q.ndim == 1
    q2 = q.reshape(1, -1) if squeeze else q
    hpk, hd = q2.shape
    out = np.zeros((hpk, hd), np.float64)
    kcol = head.kcol if head.frozen else None
    vcol = head.vcol if head.frozen else None
    z = _sinks(sinks, hpk)
    _load().orc_attend_q8_ex(head.n, hd, hpk, _p(q2), _p(head.kq), _p(head.ks), _p(kcol),
                             _p(head.vq), _p(head.vs), _p(vcol), int(first), float(softcap), _p(z), _p(out))
    return out[0] if squeeze else out


def attend_i8(q, head: I8Head, first: int = 0, sinks=None) -> np.ndarray:
    """[P3] decode_attention_int8 for one KV head: q [hpk][hd] quantised per
    head, exact integer dots scaled by qscale * kscale / sqrt(hd), softmax,
    V dequantised per row; float64.  first / sinks [hpk] as attend_f32 (the
    page's int8 route has neither; they serve as test identities)."""
    q = _f32(q)
    squeeze = q.ndim == 1
    q2 = q.reshape(1, -1) if squeeze else q
    hpk, hd = q2.shape
    out = np.zeros((hpk, hd), np.float64)
    z = None if sinks is None else _f32(np.asarray(sinks).reshape(hpk))
    _load().orc_attend_i8_ex(head.n, hd, hpk, _p(q2), _p(head.kq), _p(head.ks), _p(head.vq), _p(head.vs),
                             int(first), _p(z), _p(out))
    return out[0] if squeeze else out


def weights_f32(q, k) -> np.ndarray:
    q, k = _f32(q), _f32(k)
    hd = q.shape[0]
    k = k.reshape(-1, hd)
    w = np.zeros(k.shape[0], np.float64)
    _load().orc_weights_f32(k.shape[0], hd, _p(q), _p(k), _p(w))
    return w


def decode(q, units, n_kv_heads: int, threads: int = 1, only=None, first=None, softcap: float = 0.0,
           sinks=None) -> np.ndarray:
    """Batched decode by definition.

    q      [B][Hq][hd] f32
    units  units[b][g] -> None (dead group or nothing stored) or
           ("f32", k [n][hd], v [n][hd]) or ("q8", Q8Head) or ("i8", I8Head)
    Returns out [B][Hq][hd] float64; Q heads h of group g = h // (Hq/Hkv)
    ([P1] attend_group), zeros for dead/empty groups.
    only   optional iterable of (b, g) pairs to compute (others left 0).
    first  optional [B] first visible row per sequence; softcap, sinks [Hq]
           as attend_f32.
    """
    q = _f32(q)
    B, Hq, hd = q.shape
    hpk = Hq // n_kv_heads
    assert hpk * n_kv_heads == Hq
    out = np.zeros((B, Hq, hd), np.float64)
    todo = list(only) if only is not None else [(b, g) for b in range(B) for g in range(n_kv_heads)]

    def run(bg):
        b, g = bg
        u = units[b][g]
        if u is None:
            return
        qg = np.ascontiguousarray(q[b, g * hpk:(g + 1) * hpk])
        f = 0 if first is None else int(first[b])
        z = None if sinks is None else np.asarray(sinks, np.float32)[g * hpk:(g + 1) * hpk]
        if u[0] == "f32":
            out[b, g * hpk:(g + 1) * hpk] = attend_f32(qg, u[1], u[2], f, softcap, z)
        elif u[0] == "i8":
            out[b, g * hpk:(g + 1) * hpk] = attend_i8(qg, u[1], f, z)
        else:
            out[b, g * hpk:(g + 1) * hpk] = attend_q8(qg, u[1], f, softcap, z)

    if threads <= 1:
        for bg in todo:
            run(bg)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, todo))
    return out


# --------------------------------------------------------------------------
# R-SWA ring cursors ([P3] RingCache::record_prefill / write_decode_step)
# --------------------------------------------------------------------------
class RingModel:
    """Cursor model of the R-SWA ring: a read-only reference block of
    ``prefill_len`` rows followed by a W-slot ring.  Keeps the explicit list
    of every token written since the prefill, so the live window can be
    compared against the physical slots."""

    def __init__(self, window: int = RING_W):
        self.W = window
        self.prefill_len: Optional[int] = None
        self.ring_len = 0
        self.ring_pos = 0
        self.writes = 0
        self.slots: list = [None] * window   # slot -> token id held
        self.tokens: list = []               # every token id written, in order
        self.epoch = 0                       # lineage: bumped by a rollback that discards writes

    def record_prefill(self, n: int) -> None:
        self.prefill_len = n
        self.ring_len = 0
        self.ring_pos = 0
        self.writes = 0
        self.slots = [None] * self.W
        self.tokens = []
        self.epoch += 1

    def write(self, token) -> int:
        """Warm-up: append at ring_len (ring_pos follows ring_len mod W);
        steady state: overwrite ring_pos, then advance it mod W."""
        if self.prefill_len is None:
            raise RuntimeError("write before record_prefill")
        if self.ring_len < self.W:
            slot = self.ring_len
            self.ring_len += 1
            self.ring_pos = self.ring_len % self.W
        else:
            slot = self.ring_pos
            self.ring_pos = (self.ring_pos + 1) % self.W
        self.slots[slot] = token
        self.tokens.append(token)
        self.writes += 1
        return slot

    def window(self) -> list:
        """Explicit live window: the last min(writes, W) tokens, in order."""
        return self.tokens[-self.W:] if self.tokens else []

    def physical(self) -> list:
        """Token ids in physical slot order over the live slots 0..ring_len-1."""
        return self.slots[: self.ring_len]

    def effective_len(self) -> int:
        return (self.prefill_len or 0) + self.ring_len

    # [P3] RingCache::checkpoint / rollback_to: a checkpoint holds the cursors
    # only; a rollback restores them if that loses no live row, and starts a
    # new lineage when it discards writes.
    def checkpoint(self) -> dict:
        return dict(prefill_len=self.prefill_len, ring_len=self.ring_len, ring_pos=self.ring_pos,
                    writes=self.writes, epoch=self.epoch)

    def rollback_to(self, cp: dict) -> None:
        if cp["prefill_len"] != self.prefill_len:
            raise ValueError("checkpoint of another prefill")
        if cp["epoch"] != self.epoch:
            raise ValueError("checkpoint of an abandoned lineage")
        if cp["writes"] > self.writes:
            raise ValueError("checkpoint from the future")
        discarded = self.writes - cp["writes"]
        if cp["ring_len"] > self.W or discarded > self.W - cp["ring_len"]:
            raise ValueError("rollback would need overwritten rows")
        self.ring_len, self.ring_pos, self.writes = cp["ring_len"], cp["ring_pos"], cp["writes"]
        self.tokens = self.tokens[: cp["writes"]]
        if discarded:
            self.epoch += 1


# --------------------------------------------------------------------------
# Query-batched verify ([P3] verify_attention)
# --------------------------------------------------------------------------
def rswa_verify(q, ref_k, ref_v, history_k, history_v, draft_k, draft_v, window: int = RING_W, kind: str = "f32"):
    """K-token verify by definition: draft query i attends, with no mask, to
    the reference rows plus the ring as it would stand after the draft
    tokens 0..i were written in order -- the last min(window, n + i + 1)
    tokens of (history ++ draft[0..i]) -- i.e. the i-th of K sequential
    decode steps; nothing is written.

    q        [K][Hq][hd] f32 draft queries
    ref_k/v  [Hkv][P][hd] f32 reference rows
    history  [Hkv][n][hd] f32: every ring token written since the prefill,
             oldest first (only the last `window` are live)
    draft    [K][Hkv][hd] f32
    kind     "f32", or "i8": the int8 mirror -- every row through
             quantize_row_i8 and the decode is decode_attention_int8 (the
             page's decode_attention with its int8 switch on)
    Returns out [K][Hq][hd] float64."""
    q = _f32(q)
    K_, Hq, hd = q.shape
    Hkv = ref_k.shape[0]
    hpk = Hq // Hkv
    out = np.zeros((K_, Hq, hd), np.float64)
    for i in range(K_):
        for g in range(Hkv):
            toks_k = np.concatenate([history_k[g], draft_k[: i + 1, g]])
            toks_v = np.concatenate([history_v[g], draft_v[: i + 1, g]])
            rows_k = np.concatenate([ref_k[g], toks_k[-window:]])
            rows_v = np.concatenate([ref_v[g], toks_v[-window:]])
            qg = q[i, g * hpk:(g + 1) * hpk]
            if kind == "i8":
                h = I8Head(cap=max(rows_k.shape[0], 1))
                h.append(rows_k, rows_v)
                out[i, g * hpk:(g + 1) * hpk] = attend_i8(qg, h)
            else:
                out[i, g * hpk:(g + 1) * hpk] = attend_f32(qg, rows_k, rows_v)
    return out


# --------------------------------------------------------------------------
# Row management around the decode ([P2] LayerKvCache::truncate_last,
# trim_window_anchored)
# --------------------------------------------------------------------------
def truncate_last(n: int, n_drop: int) -> int:
    """Rows kept after dropping the last n_drop of n (never below 0)."""
    return n - min(n_drop, n)


def trim_window(base: int, n: int, w: int, slack: int, align: int, anchor: Optional[int] = None,
                q8_unfrozen: bool = False) -> int:
    """Rows a sliding-window trim drops from the front of a sequence whose
    row 0 is absolute position `base` and which stores n rows: nothing while
    n <= 2w (or w == 0, or a q8 field not frozen yet); otherwise the front is
    cut so that w + slack rows (and, with an anchor, every row from
    anchor - w - slack on) stay, the new base rounded down to a multiple of
    align."""
    if w == 0 or n <= 2 * w or q8_unfrozen:
        return 0
    align = max(align, 1)
    keep_from = max(base + n - (w + slack), 0)
    if anchor is not None:
        keep_from = min(keep_from, max(anchor - (w + slack), 0))
    new_base = keep_from // align * align
    return new_base - base if new_base > base else 0
