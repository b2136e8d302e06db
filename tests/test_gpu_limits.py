"""GPU: the library at its size limits, through the C ABI and against the
oracle -- a sequence filled to KVQ_MAX_CAPACITY rows (2^24: the largest row
offset the kernels address), the largest head count (64 KV heads with 8 Q
heads each) and a batch that spans three launches."""
import math

import numpy as np
import pytest
import torch

import oracle
from int8_kv_cache_decode_amd import kvq as K
from gpu_cases import F32_TOL, THREADS, append_rows, dev, host, max_err, oracle_q8_heads, say

pytestmark = pytest.mark.gpu

APPEND = {K.KIND_F32: K.kv_append_f32, K.KIND_Q8: K.kv_append_q8, K.KIND_I8: K.kv_append_i8}
DECODE = {K.KIND_F32: K.decode_attn_f32, K.KIND_Q8: K.decode_attn_q8, K.KIND_I8: K.decode_attn_i8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


def rng(seed):
    return np.random.default_rng(seed)


def units_for(kind, k, v, alive, cap):
    """Oracle units [g] for rows k, v [n][Hkv][128] of one sequence."""
    hkv = k.shape[1]
    if kind == K.KIND_Q8:
        heads = oracle_q8_heads(k, v, alive, cap=cap)
        return [("q8", heads[g]) if alive[g] else None for g in range(hkv)]
    out = []
    for g in range(hkv):
        if not alive[g]:
            out.append(None)
        elif kind == K.KIND_F32:
            out.append(("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g])))
        else:
            h = oracle.I8Head(cap=cap)
            h.append(k[:, g], v[:, g])
            out.append(("i8", h))
    return out


def zero_filled_case(kind, cap, alive, hpk, seed, check_window=True):
    """One sequence of cap rows: 64 random rows, zero rows, then a 4096-row
    random window at the top of the row range.  A zero row scores 0 and
    carries a zero value, so the full decode equals the oracle's decode of
    the 64 + 4096 random rows with a value-less logit ln(#zero rows) per Q
    head; the windowed decode (first = cap - 4096) sees the top rows only.
    The top rows' storage of the last live head is compared bit for bit."""
    W, H0 = 4096, 64
    hkv = len(alive)
    r = rng(seed)
    c = K.KvCache(kind, 1, hkv, cap, alive=alive)
    head_k, head_v = r.standard_normal((2, H0, hkv, 128)).astype(np.float32)
    win_k = (r.standard_normal((W, hkv, 128)) * 2).astype(np.float32)
    win_v = r.standard_normal((W, hkv, 128)).astype(np.float32)
    fn = APPEND[kind]
    fn(c, 0, H0, dev(head_k), dev(head_v))
    chunk = 1 << 20
    zeros = torch.zeros((chunk, hkv, 128), device="cuda")
    n_zero = cap - H0 - W
    left = n_zero
    while left > 0:
        n = min(left, chunk)
        fn(c, 0, n, zeros, zeros)
        left -= n
    fn(c, 0, W, dev(win_k), dev(win_v))
    torch.cuda.synchronize()
    del zeros
    assert int(c.len[0]) == cap
    rows_k, rows_v = np.concatenate([head_k, win_k]), np.concatenate([head_v, win_v])
    units = [units_for(kind, rows_k, rows_v, alive, H0 + W)]
    g = int(np.flatnonzero(alive)[-1])
    sl = int(alive[:g].sum())                      # its live slot
    u = units[0][g]
    top = slice(cap - W, cap)
    if kind == K.KIND_F32:
        assert np.array_equal(host(c.view("k")[0, sl, top]), win_k[:, g])
        assert np.array_equal(host(c.view("v")[0, sl, top]), win_v[:, g])
    else:
        h = u[1]
        for nm, want in (("kq", h.kq), ("ks", h.ks), ("vq", h.vq), ("vs", h.vs)):
            got = host(c.view(nm)[0, sl, top])
            assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(want[H0:H0 + W]).view(np.uint8)), nm
        if kind == K.KIND_Q8:
            assert int(c.frozen[0]) == 1
            assert np.array_equal(host(c.view("kcol")[0, sl]).view(np.uint32), h.kcol.view(np.uint32))
            assert np.array_equal(host(c.view("vcol")[0, sl]).view(np.uint32), h.vcol.view(np.uint32))
    hq = hkv * hpk
    q = (r.standard_normal((1, hq, 128)) * 2).astype(np.float32)
    out = torch.full((1, hq, 128), np.nan, device="cuda")
    DECODE[kind](c, hq, dev(q), out)
    torch.cuda.synchronize()
    got = host(out)
    ref = oracle.decode(q, units, hkv, threads=THREADS, sinks=np.full(hq, math.log(n_zero), np.float32))
    err = max_err(got, ref)
    say("  full context max err %.3g (|out| up to %.2f)" % (err, np.abs(ref).max()))
    assert err <= F32_TOL, err
    for gd in np.flatnonzero(alive == 0):
        assert not got[0, gd * hpk:(gd + 1) * hpk].any()
    if kind != K.KIND_I8 and check_window:
        ex = K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex
        out2 = torch.full((1, hq, 128), np.nan, device="cuda")
        ex(c, hq, dev(q), out2, K.DecodeOpts(first=np.array([cap - W], np.int32)))
        torch.cuda.synchronize()
        ref2 = oracle.decode(q, units, hkv, threads=THREADS, first=[H0])
        err2 = max_err(host(out2), ref2)
        say("  top-window max err %.3g" % err2)
        assert err2 <= F32_TOL, err2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_sequence_at_max_capacity(kind):
    """2^24 rows in one (sequence, head), the largest row offset the kernels
    address, built as in zero_filled_case (one dead and one live KV head, 4 Q
    heads each)."""
    say("case: max capacity kind", kind, "rows", K.MAX_CAPACITY)
    zero_filled_case(kind, K.MAX_CAPACITY, np.array([0, 1], np.uint8), 4, 900 + kind)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind", [K.KIND_Q8, K.KIND_I8])
def test_group_of_8_long_launch(kind):
    """Groups of 8 Q heads over 4 KV heads x 2^20 rows (262144 16-row tiles,
    more than 48 per resident wave, so the value pass runs on the matrix
    cores; shorter launches, as in the other group-of-8 tests, run it on the
    VALU), built as in zero_filled_case."""
    say("case: group of 8, long launch, kind", kind)
    zero_filled_case(kind, 1 << 20, np.ones(4, np.uint8), 8, 950 + kind)


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_max_heads(kind):
    """64 KV heads (the most a cache holds), 8 Q heads each, every 7th group
    dead; an empty sequence and a 300-row one."""
    say("case: max heads kind", kind)
    r = rng(950 + kind)
    hkv, hpk, lens = K.MAX_KV_HEADS, 8, [0, 300]
    alive = np.array([0 if g % 7 == 3 else 1 for g in range(hkv)], np.uint8)
    c = K.KvCache(kind, len(lens), hkv, max(lens), alive=alive)
    units = []
    for b, n in enumerate(lens):
        k = (r.standard_normal((n, hkv, 128)) * 1.5).astype(np.float32)
        v = r.standard_normal((n, hkv, 128)).astype(np.float32)
        if n:
            append_rows(c, b, k, v, chunks=[100])
            units.append(units_for(kind, k, v, alive, n))
        else:
            units.append([None] * hkv)
    hq = hkv * hpk
    q = r.standard_normal((len(lens), hq, 128)).astype(np.float32)
    out = torch.full((len(lens), hq, 128), np.nan, device="cuda")
    DECODE[kind](c, hq, dev(q), out)
    torch.cuda.synchronize()
    got = host(out)
    err = max_err(got, oracle.decode(q, units, hkv, threads=THREADS))
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
    assert not got[0].any()
    for g in np.flatnonzero(alive == 0):
        assert not got[:, g * hpk:(g + 1) * hpk].any()


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_batch_of_three_launches(kind):
    """300 sequences (three launches of at most 128) of ragged lengths
    0..200, two KV heads, two Q heads each."""
    say("case: 300 sequences kind", kind)
    r = rng(970 + kind)
    lens = [int(x) for x in r.integers(0, 201, 300)]
    lens[0], lens[127], lens[128], lens[299] = 0, 200, 1, 64
    hkv, hpk = 2, 2
    alive = np.array([1, 1], np.uint8)
    c = K.KvCache(kind, len(lens), hkv, max(lens), alive=alive)
    units = []
    for b, n in enumerate(lens):
        k = r.standard_normal((n, hkv, 128)).astype(np.float32)
        v = r.standard_normal((n, hkv, 128)).astype(np.float32)
        if n:
            append_rows(c, b, k, v)
            units.append(units_for(kind, k, v, alive, n))
        else:
            units.append([None] * hkv)
    hq = hkv * hpk
    q = r.standard_normal((len(lens), hq, 128)).astype(np.float32)
    out = torch.full((len(lens), hq, 128), np.nan, device="cuda")
    DECODE[kind](c, hq, dev(q), out)
    torch.cuda.synchronize()
    got = host(out)
    err = max_err(got, oracle.decode(q, units, hkv, threads=THREADS))
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
    assert not got[0].any()
