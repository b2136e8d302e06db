"""C-ABI library checks that need no GPU: it loads, exports every entry
point include/kvq.h declares, validates arguments on the host before
touching anything (a refused call leaves the host counters unchanged), and
accounts memory as the pages do.  Device pointers here are fake aligned
addresses that a refused call never dereferences."""
import ctypes
import os
import re

import numpy as np
import pytest

from int8_kv_cache_decode_amd import kvq as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"kv_append_f32", "kv_append_q8", "kv_freeze_col_and_requant", "decode_attn_f32",
            "decode_attn_q8", "rswa_decode"} <= set(names)
    lib = ctypes.CDLL(K.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    bound = {s[0] for s in K._SIGNATURES}
    assert set(names) == bound, set(names) ^ bound


def fake_cache(kind, batch=2, hkv=8, cap=256, alive=None):
    c = K.KvCache(kind, batch, hkv, cap, alive=alive, allocate=False)
    names = {K.KIND_F32: ("k", "v"), K.KIND_Q8: ("kq", "ks", "vq", "vs", "kcol", "vcol"),
             K.KIND_I8: ("kq", "ks", "vq", "vs")}[kind]
    for i, n in enumerate(names):
        setattr(c.c, n, FAKE + 4096 * i)
    return c


def snapshot(c, rings=None):
    s = (c.len.copy(), c.frozen.copy(), bytes(c.c))
    if rings is not None:
        s += (bytes(rings.arr),)
    return s


def call(fn, *args):
    return getattr(K.lib(), fn)(*args)


def expect(rc, code, c, before, rings=None):
    assert rc == code, (rc, K.last_error())
    assert K.last_error()
    after = snapshot(c, rings)
    for a, b in zip(before, after):
        assert np.array_equal(np.frombuffer(a, np.uint8) if isinstance(a, bytes) else a,
                              np.frombuffer(b, np.uint8) if isinstance(b, bytes) else b)


def test_cache_init_validation():
    c = K.kvq_cache()
    ln = np.zeros(2, np.int32)
    fr = np.zeros(2, np.uint8)
    L = K.lib()
    assert L.kvq_cache_init(ctypes.byref(c), 4, 2, 8, 128, 16, None, ln.ctypes.data, fr.ctypes.data) == K.EINVAL
    assert L.kvq_cache_init(ctypes.byref(c), 1, 2, 8, 64, 16, None, ln.ctypes.data, fr.ctypes.data) == K.EINVAL
    assert L.kvq_cache_init(ctypes.byref(c), 1, 0, 8, 128, 16, None, ln.ctypes.data, fr.ctypes.data) == K.EINVAL
    assert L.kvq_cache_init(ctypes.byref(c), 1, 2, 65, 128, 16, None, ln.ctypes.data, fr.ctypes.data) == K.EINVAL
    # capacity 1..2^24 (offsets inside a head block are 32-bit)
    assert L.kvq_cache_init(ctypes.byref(c), 2, 2, 8, 128, 0, None, ln.ctypes.data, fr.ctypes.data) == K.EINVAL
    assert L.kvq_cache_init(ctypes.byref(c), 2, 2, 8, 128, (1 << 24) + 1, None, ln.ctypes.data,
                            fr.ctypes.data) == K.EINVAL
    assert L.kvq_cache_init(ctypes.byref(c), 2, 1, 1, 128, 1 << 24, None, ln.ctypes.data, fr.ctypes.data) == K.OK
    assert L.kvq_cache_init(ctypes.byref(c), 1, 2, 8, 128, 16, None, None, fr.ctypes.data) == K.EINVAL
    alive = np.array([1, 1, 0, 1, 1, 0, 1, 1], np.uint8)
    assert L.kvq_cache_init(ctypes.byref(c), 2, 2, 8, 128, 16, alive.ctypes.data,
                            ln.ctypes.data, fr.ctypes.data) == K.OK
    assert c.n_live == 6 and list(c.live_slot[:8]) == [0, 1, -1, 2, 3, -1, 4, 5]


def test_append_refusals_leave_cache_unchanged():
    for kind, fn in ((K.KIND_F32, "kv_append_f32"), (K.KIND_Q8, "kv_append_q8")):
        c = fake_cache(kind, cap=100)
        c.len[:] = [90, 5]
        before = snapshot(c)
        expect(call(fn, c.ref, 0, 11, FAKE, FAKE, None), K.ECAPACITY, c, before)
        expect(call(fn, c.ref, 2, 1, FAKE, FAKE, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, -2, 1, FAKE, FAKE, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, 1, -1, FAKE, FAKE, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, 1, 3, None, FAKE, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, 1, 3, FAKE + 4, FAKE, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, K.ALL_SEQS, 2, FAKE, FAKE, None), K.EINVAL, c, before)
        c.len[:] = [100, 5]
        before = snapshot(c)
        expect(call(fn, c.ref, K.ALL_SEQS, 1, FAKE, FAKE, None), K.ECAPACITY, c, before)
    # wrong kind
    c = fake_cache(K.KIND_F32)
    before = snapshot(c)
    expect(call("kv_append_q8", c.ref, 0, 1, FAKE, FAKE, None), K.ESTATE, c, before)
    expect(call("kv_freeze_col_and_requant", c.ref, 0, None), K.ESTATE, c, before)
    c = fake_cache(K.KIND_Q8)
    before = snapshot(c)
    expect(call("kv_append_f32", c.ref, 0, 1, FAKE, FAKE, None), K.ESTATE, c, before)
    expect(call("kv_freeze_col_and_requant", c.ref, 5, None), K.EINVAL, c, before)


def test_missing_or_misaligned_buffers_refused():
    c = fake_cache(K.KIND_Q8)
    c.c.vs = 0
    before = snapshot(c)
    expect(call("kv_append_q8", c.ref, 0, 1, FAKE, FAKE, None), K.EINVAL, c, before)
    c = fake_cache(K.KIND_F32)
    c.c.k = FAKE + 8
    before = snapshot(c)
    expect(call("decode_attn_f32", c.ref, 8, FAKE, FAKE, FAKE, 1 << 30, None), K.EINVAL, c, before)


def test_decode_refusals():
    for kind, fn in ((K.KIND_F32, "decode_attn_f32"), (K.KIND_Q8, "decode_attn_q8")):
        c = fake_cache(kind)
        c.len[:] = [10, 20]
        need = K.kvq_workspace_bytes(c, 32)
        assert need > 0 and need % 256 == 0
        before = snapshot(c)
        expect(call(fn, c.ref, 30, FAKE, FAKE, FAKE, need, None), K.EINVAL, c, before)     # 30 % 8
        expect(call(fn, c.ref, 8 * 16, FAKE, FAKE, FAKE, 1 << 40, None), K.EINVAL, c, before)  # group 16
        expect(call(fn, c.ref, 32, None, FAKE, FAKE, need, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, 32, FAKE, FAKE, None, need, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, 32, FAKE, FAKE, FAKE, need - 1, None), K.EINVAL, c, before)
        c.len[1] = 300                                     # len beyond capacity
        before = snapshot(c)
        expect(call(fn, c.ref, 32, FAKE, FAKE, FAKE, need, None), K.ESTATE, c, before)
    c = fake_cache(K.KIND_Q8)
    before = snapshot(c)
    expect(call("decode_attn_f32", c.ref, 32, FAKE, FAKE, FAKE, 1 << 40, None), K.ESTATE, c, before)


def test_decode_option_refusals():
    """decode_attn_*_ex refuse bad options before any launch: a negative
    first row, a negative or non-finite soft-cap, reserved != 0."""
    for kind, fn in ((K.KIND_F32, "decode_attn_f32_ex"), (K.KIND_Q8, "decode_attn_q8_ex")):
        c = fake_cache(kind)
        c.len[:] = [10, 20]
        need = K.kvq_workspace_bytes(c, 32)
        before = snapshot(c)
        for first, cap, res in (([0, -1], 0.0, 0), (None, -1.0, 0), (None, float("nan"), 0),
                                (None, float("inf"), 0), (None, 0.0, 1)):
            o = K.DecodeOpts(first=first, softcap=cap)
            o.c.reserved = res
            expect(call(fn, c.ref, 32, FAKE, FAKE, o.ref, FAKE, need, None), K.EINVAL, c, before)
        # the usual argument checks come first and still apply
        o = K.DecodeOpts(first=[0, 0], softcap=30.0)
        expect(call(fn, c.ref, 30, FAKE, FAKE, o.ref, FAKE, need, None), K.EINVAL, c, before)
        expect(call(fn, c.ref, 32, FAKE, FAKE, o.ref, FAKE, need - 1, None), K.EINVAL, c, before)
    c = fake_cache(K.KIND_Q8)
    before = snapshot(c)
    expect(call("decode_attn_f32_ex", c.ref, 32, FAKE, FAKE, None, FAKE, 1 << 40, None), K.ESTATE, c, before)


def test_verify_refusals():
    """rswa_verify refuses before any launch: bad counts, too many queries
    per KV head, a small workspace, an unrecorded prefill, a q8 cache."""
    c = fake_cache(K.KIND_F32, batch=2, hkv=10, cap=400)
    rings = K.Rings(2)
    c.len[:] = [5, 5]
    need = K.kvq_verify_workspace_bytes(c, 10, 4)
    assert need > 0 and K.kvq_verify_workspace_bytes(c, 10, 17) == 0 and K.kvq_verify_workspace_bytes(c, 20, 9) == 0
    before = snapshot(c, rings)
    expect(call("rswa_verify", c.ref, rings.ref, 10, 4, FAKE, FAKE, FAKE, FAKE, FAKE, need, None), K.ESTATE,
           c, before, rings)                                            # prefill not recorded
    K.rswa_record_prefill(c, rings, 0)
    K.rswa_record_prefill(c, rings, 1)
    before = snapshot(c, rings)
    for n_q, n_d, ws in ((10, 0, need), (10, 17, 1 << 40), (20, 9, 1 << 40), (15, 1, 1 << 40), (10, 4, need - 1)):
        expect(call("rswa_verify", c.ref, rings.ref, n_q, n_d, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None), K.EINVAL,
               c, before, rings)
    expect(call("rswa_verify", c.ref, rings.ref, 10, 4, None, FAKE, FAKE, FAKE, FAKE, need, None), K.EINVAL,
           c, before, rings)
    c.len[1] = 6                                                        # appended since the record
    before = snapshot(c, rings)
    expect(call("rswa_verify", c.ref, rings.ref, 10, 4, FAKE, FAKE, FAKE, FAKE, FAKE, need, None), K.ESTATE,
           c, before, rings)
    q = fake_cache(K.KIND_Q8)
    bq = snapshot(q)
    expect(call("rswa_verify", q.ref, rings.ref, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None), K.ESTATE, q, bq)


def test_truncate_last_moves_the_cursor_only():
    """[P1]/[P2] truncate_last: drop the last min(n_drop, len) rows."""
    c = fake_cache(K.KIND_Q8, batch=3)
    c.len[:] = [10, 3, 0]
    c.frozen[:] = [1, 0, 0]
    K.kv_truncate_last(c, 0, 4)
    assert list(c.len) == [6, 3, 0] and list(c.frozen) == [1, 0, 0]
    K.kv_truncate_last(c, K.ALL_SEQS, 5)
    assert list(c.len) == [1, 0, 0]
    before = snapshot(c)
    expect(call("kv_truncate_last", c.ref, 0, -1), K.EINVAL, c, before)
    expect(call("kv_truncate_last", c.ref, 3, 1), K.EINVAL, c, before)


def test_trim_window_no_op_cases_and_refusals():
    """[P2] trim_window: nothing while len <= 2w, for w == 0, on a q8
    sequence whose field is not frozen, or when the rounded cut does not pass
    the base; bad arguments are refused with nothing changed.  (Trims that
    move rows run on the GPU.)"""
    c = fake_cache(K.KIND_F32, batch=2, cap=256)
    c.len[:] = [20, 21]
    assert K.kv_trim_window(c, 0, 0, 10, 2, 4, stream=0) == (0, 0)          # 20 <= 2w
    assert K.kv_trim_window(c, 1, 0, 0, 2, 4, stream=0) == (0, 0)           # w == 0
    assert K.kv_trim_window(c, 1, 12, 10, 2, 32, stream=0) == (12, 0)       # cut rounds down to 0 <= base
    q = fake_cache(K.KIND_Q8, batch=1, cap=256)
    q.len[:] = [200]
    assert K.kv_trim_window(q, 0, 0, 10, 2, 4, stream=0) == (0, 0)          # field not frozen
    assert list(c.len) == [20, 21] and list(q.len) == [200]
    base = ctypes.c_int64(0)
    before = snapshot(c)
    expect(call("kv_trim_window", c.ref, 0, None, 5, 1, 1, -1, None, 0), K.EINVAL, c, before)
    expect(call("kv_trim_window", c.ref, 2, ctypes.byref(base), 5, 1, 1, -1, None, 0), K.EINVAL, c, before)
    for w, sl, al in ((-1, 1, 1), (5, -1, 1), (5, 1, -1)):
        expect(call("kv_trim_window", c.ref, 0, ctypes.byref(base), w, sl, al, -1, None, 0), K.EINVAL, c, before)
    base = ctypes.c_int64(-3)
    expect(call("kv_trim_window", c.ref, 0, ctypes.byref(base), 5, 1, 1, -1, None, 0), K.EINVAL, c, before)
    # every sequence at once: one base per sequence; a negative one is refused
    # before anything changes, no-op rows report 0 dropped
    bases = (ctypes.c_int64 * 2)(0, -1)
    expect(call("kv_trim_window", c.ref, K.ALL_SEQS, bases, 5, 1, 1, -1, None, 0), K.EINVAL, c, before)
    assert list(bases) == [0, -1]
    nb, nd = K.kv_trim_window(c, K.ALL_SEQS, [0, 12], 10, 2, 32, stream=0)   # no sequence trims
    assert list(nb) == [0, 12] and list(nd) == [0, 0] and list(c.len) == [20, 21]


def test_ring_checkpoint_and_rollback_cursors():
    """[P3] checkpoint / rollback_to on the host cursors, the page's 9-accept,
    6-draft example; a no-op rollback keeps the lineage; a re-prefill starts
    a new one."""
    c = fake_cache(K.KIND_F32, batch=2, hkv=10, cap=400)
    rings = K.Rings(2)
    c.len[:] = [5, 0]
    K.rswa_record_prefill(c, rings, 0)
    e0 = rings[0].epoch
    r = rings[0]
    r.ring_len, r.ring_pos, r.writes = 9, 9, 9              # 9 accepted steps
    c.len[0] = 14
    cp = K.rswa_checkpoint(c, rings, 0)
    assert (cp.prefill_len, cp.ring_len, cp.ring_pos, cp.writes, cp.epoch, cp.seq) == (5, 9, 9, 9, e0, 0)
    r.ring_len, r.ring_pos, r.writes = 15, 15, 15           # 6 draft steps
    c.len[0] = 20
    K.rswa_rollback_to(c, rings, 0, cp)
    assert (r.ring_len, r.ring_pos, r.writes, c.len[0]) == (9, 9, 9, 14) and r.epoch == e0 + 1
    cp2 = K.rswa_checkpoint(c, rings, 0)
    K.rswa_rollback_to(c, rings, 0, cp2)                    # nothing discarded: identity
    assert (r.ring_len, r.writes, r.epoch, c.len[0]) == (9, 9, e0 + 1, 14)
    K.rswa_record_prefill(c, rings, 1)
    assert rings[1].epoch == 1


def test_ring_rollback_refusals_leave_everything_unchanged():
    """[P3] rollback_to refusals: another cache, another sequence, a stale
    lineage, a checkpoint from the future, and discarded writes that wrapped
    onto slots live at the checkpoint (steady state)."""
    c = fake_cache(K.KIND_F32, batch=2, hkv=10, cap=400)
    other = fake_cache(K.KIND_F32, batch=2, hkv=10, cap=400)
    rings, orings = K.Rings(2), K.Rings(2)
    c.len[:] = [3, 3]
    other.len[:] = [3, 3]
    for b in range(2):
        K.rswa_record_prefill(c, rings, b)
        K.rswa_record_prefill(other, orings, b)
    r = rings[0]
    r.ring_len, r.ring_pos, r.writes = 128, 0, 128          # ring just full
    c.len[0] = 131
    cp_full = K.rswa_checkpoint(c, rings, 0)
    r.ring_pos, r.writes = 1, 129                           # one steady-state write
    before = snapshot(c, rings)
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, ctypes.byref(cp_full)), K.ESTATE, c, before, rings)
    foreign = K.rswa_checkpoint(other, orings, 0)
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, ctypes.byref(foreign)), K.ESTATE, c, before, rings)
    seq1 = K.rswa_checkpoint(c, rings, 1)
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, ctypes.byref(seq1)), K.ESTATE, c, before, rings)
    cp = K.rswa_checkpoint(c, rings, 0)
    fut = K.kvq_ring_checkpoint.from_buffer_copy(cp)
    fut.writes += 1
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, ctypes.byref(fut)), K.ESTATE, c, before, rings)
    stale = K.kvq_ring_checkpoint.from_buffer_copy(cp)
    stale.epoch -= 1
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, ctypes.byref(stale)), K.ESTATE, c, before, rings)
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, None), K.EINVAL, c, before, rings)
    q = fake_cache(K.KIND_Q8)
    bq = snapshot(q)
    expect(call("rswa_checkpoint", q.ref, rings.ref, 0, ctypes.byref(cp)), K.ESTATE, q, bq)


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
def test_rswa_refusals_leave_cache_and_rings_unchanged(kind):
    """The same refusals on f32 caches and on the per-row int8 kind (the
    page's int8 mirror shares the ring layout); q8 caches hold no ring."""
    q = fake_cache(K.KIND_Q8, batch=2, hkv=10, cap=200)
    qr = K.Rings(2)
    bq = snapshot(q, qr)
    expect(call("rswa_record_prefill", q.ref, qr.ref, 0), K.ESTATE, q, bq, qr)
    expect(call("rswa_decode", q.ref, qr.ref, 10, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None), K.ESTATE,
           q, bq, qr)
    c = fake_cache(kind, batch=2, hkv=10, cap=200)
    rings = K.Rings(2)
    ws = K.kvq_workspace_bytes(c, 10)
    before = snapshot(c, rings)
    # decode before record_prefill ([P3] decode_before_prefill_errors)
    expect(call("rswa_decode", c.ref, rings.ref, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None), K.ESTATE,
           c, before, rings)
    c.len[:] = [73, 72]
    before = snapshot(c, rings)
    # prefill + W beyond capacity
    expect(call("rswa_record_prefill", c.ref, rings.ref, 0), K.ECAPACITY, c, before, rings)
    expect(call("rswa_record_prefill", c.ref, rings.ref, 2), K.EINVAL, c, before, rings)
    assert call("rswa_record_prefill", c.ref, rings.ref, 1) == K.OK
    assert rings[1].prefill_len == 72 and rings[1].ring_len == 0 and rings[1].ring_pos == 0
    c.len[0] = 10
    assert call("rswa_record_prefill", c.ref, rings.ref, 0) == K.OK
    before = snapshot(c, rings)
    # malformed steps must not write ([P3] malformed q/k/v do not mutate)
    expect(call("rswa_decode", c.ref, rings.ref, 10, FAKE, None, FAKE, FAKE, FAKE, ws, None), K.EINVAL,
           c, before, rings)
    expect(call("rswa_decode", c.ref, rings.ref, 10, None, FAKE, FAKE, FAKE, FAKE, ws, None), K.EINVAL,
           c, before, rings)
    expect(call("rswa_decode", c.ref, rings.ref, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 256, None),
           K.EINVAL, c, before, rings)
    expect(call("rswa_decode", c.ref, rings.ref, 15, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None), K.EINVAL,
           c, before, rings)
    # the sequence was appended to after its prefill was recorded
    c.len[0] = 11
    before = snapshot(c, rings)
    expect(call("rswa_decode", c.ref, rings.ref, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None), K.ESTATE,
           c, before, rings)


def test_buffer_and_workspace_sizes():
    c = fake_cache(K.KIND_Q8, batch=3, hkv=8, cap=1000, alive=[1, 1, 0, 1, 1, 0, 1, 1])
    rows = 3 * 6 * 1000
    # K codes are tile-major: each (sequence, live head) holds whole 16-row tiles
    assert K.kvq_buffer_bytes(c, K.BUF_KQ) == 3 * 6 * 1008 * 128
    assert K.kvq_buffer_bytes(c, K.BUF_KS) == rows * 16
    assert K.kvq_buffer_bytes(c, K.BUF_VQ) == rows * 128
    assert K.kvq_buffer_bytes(c, K.BUF_VS) == rows * 4
    assert K.kvq_buffer_bytes(c, K.BUF_KCOL) == 3 * 6 * 512
    assert K.kvq_buffer_bytes(c, K.BUF_K) == 0
    f = fake_cache(K.KIND_F32, batch=3, hkv=8, cap=1000, alive=[1, 1, 0, 1, 1, 0, 1, 1])
    assert K.kvq_buffer_bytes(f, K.BUF_K) == rows * 512 and K.kvq_buffer_bytes(f, K.BUF_KQ) == 0
    assert K.kvq_workspace_bytes(c, 30) == 0 and K.kvq_workspace_bytes(c, 32) > 0


def test_i8_kind_buffers_and_refusals():
    """The per-row int8 kind: one scale per row for K and for V, no column
    fields, 264 B per (row, head); calls of the other kinds refuse it."""
    c = fake_cache(K.KIND_I8, batch=3, hkv=8, cap=1000, alive=[1, 1, 0, 1, 1, 0, 1, 1])
    rows = 3 * 6 * 1000
    assert K.kvq_buffer_bytes(c, K.BUF_KQ) == 3 * 6 * 1008 * 128 and K.kvq_buffer_bytes(c, K.BUF_VQ) == rows * 128
    assert K.kvq_buffer_bytes(c, K.BUF_KS) == rows * 4 and K.kvq_buffer_bytes(c, K.BUF_VS) == rows * 4
    c16 = fake_cache(K.KIND_I8, batch=1, hkv=2, cap=1024)
    assert K.kvq_buffer_bytes(c16, K.BUF_KQ) == K.kvq_buffer_bytes(c16, K.BUF_VQ) == 2 * 1024 * 128
    assert K.kvq_buffer_bytes(c, K.BUF_KCOL) == 0 and K.kvq_buffer_bytes(c, K.BUF_K) == 0
    c.len[:] = [2, 0, 0]
    assert K.kvq_cache_bytes(c) == 2 * 6 * 264
    before = snapshot(c)
    expect(call("kv_append_q8", c.ref, 0, 1, FAKE, FAKE, None), K.ESTATE, c, before)
    expect(call("decode_attn_q8", c.ref, 16, FAKE, FAKE, FAKE, 1 << 40, None), K.ESTATE, c, before)
    expect(call("kv_append_i8", c.ref, 0, 999, FAKE, FAKE, None), K.ECAPACITY, c, before)
    expect(call("kv_append_i8", c.ref, 3, 1, FAKE, FAKE, None), K.EINVAL, c, before)
    expect(call("decode_attn_i8", c.ref, 12, FAKE, FAKE, FAKE, 1 << 40, None), K.EINVAL, c, before)  # 12 % 8
    f = fake_cache(K.KIND_F32)
    bf = snapshot(f)
    expect(call("decode_attn_i8", f.ref, 16, FAKE, FAKE, FAKE, 1 << 40, None), K.ESTATE, f, bf)


def test_memory_accounting_matches_pages():
    """[P1] test append_tracks_seq_len_and_layout / dead_head_stores_nothing,
    scaled to head_dim 128: one f32 row of a live head is 2*4*128 bytes and a
    dead head stores nothing; q8_2f is 276 B per (row, head) plus the frozen
    column fields -> the x3.71 ratio the pages quote as "~3.7"."""
    f = fake_cache(K.KIND_F32, batch=1, hkv=2, cap=64, alive=[1, 0])
    f.len[0] = 2
    assert K.kvq_cache_bytes(f) == 2 * 2 * 128 * 4
    q = fake_cache(K.KIND_Q8, batch=1, hkv=2, cap=64, alive=[1, 0])
    q.len[0] = 2
    assert K.kvq_cache_bytes(q) == 2 * 276
    q.frozen[0] = 1
    assert K.kvq_cache_bytes(q) == 2 * 276 + 2 * 128 * 4
    big_f = fake_cache(K.KIND_F32, batch=1, hkv=8, cap=1 << 20)
    big_q = fake_cache(K.KIND_Q8, batch=1, hkv=8, cap=1 << 20)
    big_f.len[0] = big_q.len[0] = 1 << 20
    big_q.frozen[0] = 1
    ratio = K.kvq_cache_bytes(big_f) / K.kvq_cache_bytes(big_q)
    assert abs(ratio - 1024 / 276) < 1e-3 and round(ratio, 1) == 3.7


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(K, "_lib", None)
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        K.lib()


def test_shared_reference_record_and_refusals():
    """rswa_shared_record_prefill / rswa_shared_decode refuse before any
    launch, leaving the cache and every stream's cursors unchanged; a record
    sets each stream's cursors and reserves its ring rows."""
    c = fake_cache(K.KIND_F32, batch=2, hkv=10, cap=2000)
    rings = K.Rings(16)
    c.len[:] = [1000, 7]
    before = snapshot(c, rings)
    expect(call("rswa_shared_record_prefill", c.ref, 0, rings.ref, 0), K.EINVAL, c, before, rings)
    expect(call("rswa_shared_record_prefill", c.ref, 0, rings.ref, 17), K.EINVAL, c, before, rings)
    expect(call("rswa_shared_record_prefill", c.ref, 2, rings.ref, 4), K.EINVAL, c, before, rings)
    expect(call("rswa_shared_record_prefill", c.ref, 0, rings.ref, 8), K.ECAPACITY, c, before, rings)   # 1000 + 1024
    q = fake_cache(K.KIND_Q8, batch=2, hkv=10, cap=2000)
    bq = snapshot(q, rings)
    expect(call("rswa_shared_record_prefill", q.ref, 0, rings.ref, 4), K.ESTATE, q, bq, rings)
    ws = K.kvq_verify_workspace_bytes(c, 10, 4)
    assert ws > 0 and K.kvq_verify_workspace_bytes(c, 10, 17) == 0
    # decode before the group was recorded
    expect(call("rswa_shared_decode", c.ref, 0, rings.ref, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None),
           K.ESTATE, c, before, rings)
    assert call("rswa_shared_record_prefill", c.ref, 0, rings.ref, 4) == K.OK
    assert c.len[0] == 1000 + 4 * 128
    assert all(rings[s].prefill_len == 1000 and rings[s].ring_len == 0 and rings[s].epoch == 1 for s in range(4))
    assert rings[4].prefill_len == -1
    before = snapshot(c, rings)
    bad = [((0, rings.ref, 9, 20), K.EINVAL),          # 9 x 2 > 16
           ((0, rings.ref, 0, 10), K.EINVAL),
           ((3, rings.ref, 4, 10), K.EINVAL),          # seq out of range
           ((0, rings.ref, 4, 15), K.EINVAL),          # not a multiple of 10
           ((0, rings.ref, 3, 10), K.ESTATE),          # len != prefill + 128 x 3
           ((0, None, 4, 10), K.EINVAL)]
    for (seq, rr, ns, hq), code in bad:
        expect(call("rswa_shared_decode", c.ref, seq, rr, ns, hq, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None),
               code, c, before, rings)
    expect(call("rswa_shared_decode", c.ref, 0, rings.ref, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 256, None),
           K.EINVAL, c, before, rings)
    expect(call("rswa_shared_decode", c.ref, 0, rings.ref, 4, 10, FAKE, None, FAKE, FAKE, FAKE, ws, None),
           K.EINVAL, c, before, rings)
    c.len[0] += 1                                       # appended to since the record
    before = snapshot(c, rings)
    expect(call("rswa_shared_decode", c.ref, 0, rings.ref, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None),
           K.ESTATE, c, before, rings)
    c.len[0] -= 1
    rings[2].ring_pos = 200                             # corrupt cursor of one stream
    before = snapshot(c, rings)
    expect(call("rswa_shared_decode", c.ref, 0, rings.ref, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None),
           K.ESTATE, c, before, rings)


def shared_group(kind=K.KIND_F32, n_streams=4, pre=100):
    c = fake_cache(kind, batch=2, hkv=10, cap=pre + 128 * 16)
    rings = K.Rings(16)
    c.len[:] = [pre, 7]
    assert call("rswa_shared_record_prefill", c.ref, 0, rings.ref, n_streams) == K.OK
    return c, rings


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
def test_shared_checkpoint_and_rollback_cursors(kind):
    """[P3] BatchedRingCache::checkpoint / rollback_to: per stream, on the
    single-stream rules; the page's 9-accept / 6-draft example on stream 2
    of 4 leaves every other stream and the reserved rows as they were."""
    c, rings = shared_group(kind)
    e0 = [rings[s].epoch for s in range(4)]
    for s in range(4):
        rings[s].ring_len, rings[s].ring_pos, rings[s].writes = 9, 9, 9
    cp = K.rswa_shared_checkpoint(c, 0, rings, 4, 2)
    assert (cp.prefill_len, cp.ring_len, cp.ring_pos, cp.writes, cp.epoch, cp.seq, cp.stream) == \
        (100, 9, 9, 9, e0[2], 0, 2)
    for s in range(4):
        rings[s].ring_len, rings[s].ring_pos, rings[s].writes = 15, 15, 15
    K.rswa_shared_rollback_to(c, 0, rings, 4, 2, cp)
    assert (rings[2].ring_len, rings[2].ring_pos, rings[2].writes, rings[2].epoch) == (9, 9, 9, e0[2] + 1)
    for s in (0, 1, 3):
        assert (rings[s].ring_len, rings[s].ring_pos, rings[s].writes, rings[s].epoch) == (15, 15, 15, e0[s])
    assert c.len[0] == 100 + 4 * 128 and c.len[1] == 7
    cp2 = K.rswa_shared_checkpoint(c, 0, rings, 4, 2)
    K.rswa_shared_rollback_to(c, 0, rings, 4, 2, cp2)          # nothing discarded: same lineage
    assert (rings[2].ring_len, rings[2].writes, rings[2].epoch) == (9, 9, e0[2] + 1)
    # steady state: a rollback of 128 - ring_len writes or fewer is lossless
    rings[1].ring_len, rings[1].ring_pos, rings[1].writes = 128, 5, 300
    cp1 = K.rswa_shared_checkpoint(c, 0, rings, 4, 1)
    rings[1].ring_pos, rings[1].writes = 6, 301
    with pytest.raises(K.KvqError):
        K.rswa_shared_rollback_to(c, 0, rings, 4, 1, cp1)


def test_shared_rollback_refusals_leave_everything_unchanged():
    """The refusals of a shared stream's rollback, each before any change:
    a checkpoint of another cache, sequence or stream, of a single-sequence
    ring (and a stream's checkpoint on rswa_rollback_to), a stale lineage,
    a checkpoint from the future, discarded writes past the free slots,
    indices out of range, a group not recorded or resized, a q8 cache."""
    c, rings = shared_group()
    other, orings = shared_group()
    for s in range(4):
        rings[s].ring_len, rings[s].ring_pos, rings[s].writes = 20, 20, 20
        orings[s].ring_len, orings[s].ring_pos, orings[s].writes = 20, 20, 20
    cp = K.rswa_shared_checkpoint(c, 0, rings, 4, 1)
    for s in range(4):
        rings[s].ring_len, rings[s].ring_pos, rings[s].writes = 30, 30, 30
    before = snapshot(c, rings)

    def refused(code, *args):
        expect(call("rswa_shared_rollback_to", c.ref, *args), code, c, before, rings)

    foreign = K.rswa_shared_checkpoint(other, 0, orings, 4, 1)
    refused(K.ESTATE, 0, rings.ref, 4, 1, ctypes.byref(foreign))
    refused(K.ESTATE, 0, rings.ref, 4, 2, ctypes.byref(cp))                 # another stream
    wrong_seq = K.kvq_ring_checkpoint.from_buffer_copy(cp)
    wrong_seq.seq = 1
    refused(K.ESTATE, 0, rings.ref, 4, 1, ctypes.byref(wrong_seq))
    single = K.kvq_ring_checkpoint.from_buffer_copy(cp)
    single.stream = -1
    refused(K.ESTATE, 0, rings.ref, 4, 1, ctypes.byref(single))
    expect(call("rswa_rollback_to", c.ref, rings.ref, 0, ctypes.byref(cp)), K.ESTATE, c, before, rings)
    for field, delta in (("epoch", -1), ("writes", 100), ("prefill_len", 1)):
        bad = K.kvq_ring_checkpoint.from_buffer_copy(cp)
        setattr(bad, field, getattr(bad, field) + delta)
        refused(K.ESTATE, 0, rings.ref, 4, 1, ctypes.byref(bad))
    wrapped = K.kvq_ring_checkpoint.from_buffer_copy(cp)
    wrapped.ring_len = 120                       # 10 discarded writes > 128 - 120 free slots
    refused(K.ESTATE, 0, rings.ref, 4, 1, ctypes.byref(wrapped))
    refused(K.EINVAL, 0, rings.ref, 4, 1, None)
    refused(K.EINVAL, 0, rings.ref, 4, 4, ctypes.byref(cp))                 # stream out of range
    refused(K.EINVAL, 0, rings.ref, 17, 1, ctypes.byref(cp))
    refused(K.EINVAL, 2, rings.ref, 4, 1, ctypes.byref(cp))                 # seq out of range
    refused(K.ESTATE, 0, rings.ref, 3, 1, ctypes.byref(cp))                 # len != prefill + 128 x 3
    refused(K.EINVAL, 0, None, 4, 1, ctypes.byref(cp))
    out = K.kvq_ring_checkpoint()
    expect(call("rswa_shared_checkpoint", c.ref, 0, rings.ref, 3, 1, ctypes.byref(out)), K.ESTATE, c, before, rings)
    expect(call("rswa_shared_checkpoint", c.ref, 0, rings.ref, 4, 1, None), K.EINVAL, c, before, rings)
    fresh = fake_cache(K.KIND_F32, batch=2, hkv=10, cap=3000)
    frings = K.Rings(4)
    fresh.len[:] = [100 + 4 * 128, 0]
    bf = snapshot(fresh, frings)
    expect(call("rswa_shared_checkpoint", fresh.ref, 0, frings.ref, 4, 0, ctypes.byref(out)), K.ESTATE,
           fresh, bf, frings)                                               # group not recorded
    q = fake_cache(K.KIND_Q8, batch=2, hkv=10, cap=3000)
    bq = snapshot(q, rings)
    expect(call("rswa_shared_rollback_to", q.ref, 0, rings.ref, 4, 1, ctypes.byref(cp)), K.ESTATE, q, bq, rings)


def test_noalloc_decode_refusals_before_any_device_work():
    """decode_attn_q8_noalloc validates like decode_attn_q8, and refuses a
    cache whose workspace would not fit its 64 MiB static array; all of it
    before the device is touched."""
    c = fake_cache(K.KIND_Q8)
    c.len[:] = [10, 20]
    before = snapshot(c)
    for args, code in (((30, FAKE, FAKE), K.EINVAL), ((8 * 16, FAKE, FAKE), K.EINVAL),
                       ((32, None, FAKE), K.EINVAL), ((32, FAKE, None), K.EINVAL), ((32, FAKE + 8, FAKE), K.EINVAL)):
        expect(call("decode_attn_q8_noalloc", c.ref, *args, None), code, c, before)
    f = fake_cache(K.KIND_F32)
    bf = snapshot(f)
    expect(call("decode_attn_q8_noalloc", f.ref, 32, FAKE, FAKE, None), K.ESTATE, f, bf)
    # group 8, 128 sequences x 64 live heads: 2 x 8192 slots x 8 heads x 520 B > 64 MiB
    big = fake_cache(K.KIND_Q8, batch=128, hkv=64, cap=16)
    assert K.kvq_workspace_bytes(big, 512) > 64 << 20
    bb = snapshot(big)
    expect(call("decode_attn_q8_noalloc", big.ref, 512, FAKE, FAKE, None), K.EINVAL, big, bb)
    assert "64" in K.last_error() or "static" in K.last_error()


def test_int8_verify_workspace_and_refusals():
    """The verify workspace holds the partial states only, for either kind:
    the int8 kind quantises its drafts inside the kernel.  A workspace one
    block short is refused untouched, and a q8 cache has no ring."""
    f = fake_cache(K.KIND_F32, batch=3, hkv=4, cap=300)
    i = fake_cache(K.KIND_I8, batch=3, hkv=4, cap=300)
    wf, wi = K.kvq_verify_workspace_bytes(f, 8, 5), K.kvq_verify_workspace_bytes(i, 8, 5)
    assert wi == wf and wi == K.kvq_workspace_bytes(i, 8 * 5)
    rings = K.Rings(3)
    for b in range(3):
        i.len[b] = 10
        assert call("rswa_record_prefill", i.ref, rings.ref, b) == K.OK
    before = snapshot(i, rings)
    expect(call("rswa_verify", i.ref, rings.ref, 8, 5, FAKE, FAKE, FAKE, FAKE, FAKE, wi - 256, None), K.EINVAL,
           i, before, rings)
    q = fake_cache(K.KIND_Q8, batch=3, hkv=4, cap=300)
    bq = snapshot(q, rings)
    expect(call("rswa_verify", q.ref, rings.ref, 8, 5, FAKE, FAKE, FAKE, FAKE, FAKE, wi, None), K.ESTATE,
           q, bq, rings)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark has no multi-GPU path: --gpus 2 exits non-zero with a
    message, before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
