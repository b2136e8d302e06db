"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: int8 codes, scales, column fields and ring slots bit-exact; f32
outputs within 1e-5 max-abs of the float64 oracle (the q8 path against the
oracle applied to the same dequantised K/V -- the oracle's own codes, which
must equal the GPU's bit for bit).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from int8_kv_cache_decode_amd import kvq as K
from gpu_cases import (F32_TOL, THREADS, append_rows, assert_codes_equal, dev, host, max_err,
                       oracle_q8_heads, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


def rng(seed):
    return np.random.default_rng(seed)


def channel_rows(r, n, hkv, lo=0.25, hi=8.0):
    """Rows [n][hkv][128] ~ N(0,1) times per-channel log-uniform factors."""
    f = np.exp(r.uniform(np.log(lo), np.log(hi), (hkv, 128)))
    return (r.standard_normal((n, hkv, 128)) * f).astype(np.float32)


# ---------------------------------------------------------------------------
# append / codec
# ---------------------------------------------------------------------------
def test_append_f32_layout():
    say("case: append_f32_layout")
    r = rng(1)
    alive = np.array([1, 0, 1, 1], np.uint8)
    c = K.KvCache(K.KIND_F32, 2, 4, 100, alive=alive)
    k0, v0 = r.standard_normal((2, 37, 4, 128)).astype(np.float32)
    append_rows(c, 0, k0, v0, chunks=[5, 25])
    kall, vall = r.standard_normal((2, 3, 2, 4, 128)).astype(np.float32)
    for t in range(3):
        K.kv_append_f32(c, K.ALL_SEQS, 1, dev(kall[t]), dev(vall[t]))
    torch.cuda.synchronize()
    assert list(c.len) == [40, 3]
    kk, vv = host(c.view("k")), host(c.view("v"))
    for slot, g in enumerate(np.flatnonzero(alive)):
        assert np.array_equal(kk[0, slot, :37], k0[:, g]) and np.array_equal(vv[0, slot, :37], v0[:, g])
        for t in range(3):
            assert np.array_equal(kk[0, slot, 37 + t], kall[t, 0, g])
            assert np.array_equal(kk[1, slot, t], kall[t, 1, g])
            assert np.array_equal(vv[1, slot, t], vall[t, 1, g])
        assert not kk[0, slot, 40:].any() and not kk[1, slot, 3:].any()


@pytest.mark.parametrize("case", ["row_by_row", "chunks", "one_call", "explicit_freeze", "short"])
def test_q8_codec_bitexact(case):
    say("case: q8_codec", case)
    r = rng({"row_by_row": 101, "chunks": 102, "one_call": 103, "explicit_freeze": 104, "short": 105}[case])
    alive = np.array([1, 1, 0, 1], np.uint8)
    n = {"row_by_row": 100, "chunks": 150, "one_call": 300, "explicit_freeze": 70, "short": 50}[case]
    k, v = channel_rows(r, n, 4), channel_rows(r, n, 4)
    c = K.KvCache(K.KIND_Q8, 1, 4, n, alive=alive)          # capacity exactly full
    if case == "row_by_row":
        append_rows(c, 0, k, v, chunks=list(range(1, n)))
    elif case == "chunks":
        append_rows(c, 0, k, v, chunks=[7, 71, 72])
    elif case == "explicit_freeze":
        append_rows(c, 0, k[:40], v[:40])
        K.kv_freeze_col_and_requant(c, 0)
        K.kv_freeze_col_and_requant(c, 0)                    # idempotent
        append_rows(c, 0, k[40:], v[40:])
    else:
        append_rows(c, 0, k, v)
    torch.cuda.synchronize()
    if case == "explicit_freeze":
        heads = oracle_q8_heads(k[:40], v[:40], alive, cap=n)
        for h in heads:
            if h is not None:
                h.freeze()
        for g, h in enumerate(heads):
            if h is not None:
                h.append(k[40:, g], v[40:, g])
    else:
        heads = oracle_q8_heads(k, v, alive, cap=n)
    assert_codes_equal(c, 0, heads, alive, n)


def test_q8_codec_fixture_rows(golden_dir):
    """The quantiser fixtures (half-away ties, divide-not-reciprocal cases,
    all-zero groups, extreme magnitudes) through the GPU codec."""
    import json
    import os
    import struct
    say("case: q8_codec_fixture_rows")
    fx = json.load(open(os.path.join(golden_dir, "q8_2f_quant_fixtures.json")))
    rows = []
    x = np.zeros(128, np.float32)
    x[: len(fx["half_away_row"]["row_prefix"])] = fx["half_away_row"]["row_prefix"]
    rows.append(x)
    for case in fx["division_cases"]["cases"]:
        y = np.zeros(128, np.float32)
        y[0] = struct.unpack("<f", struct.pack("<I", int(case["absmax_bits"], 16)))[0]
        y[1] = struct.unpack("<f", struct.pack("<I", int(case["x_bits"], 16)))[0]
        rows.append(y)
    r = rng(5)
    rows.append(np.zeros(128, np.float32))
    rows.append((r.standard_normal(128) * 1e-14).astype(np.float32))     # scale floor 1e-12
    rows.append((r.standard_normal(128) * 1e15).astype(np.float32))
    ints = r.integers(-127, 128, 128).astype(np.float32)
    ints[::32] = 127
    rows.append(ints)
    base = np.stack(rows)                                                 # [m][128]
    reps = -(-100 // len(base))
    kv = np.tile(base, (reps, 1))[:100]
    k = np.stack([kv, kv[::-1]], axis=1).astype(np.float32)              # [100][2][128]
    v = np.stack([kv[::-1], kv], axis=1).astype(np.float32)
    c = K.KvCache(K.KIND_Q8, 1, 2, 100)
    append_rows(c, 0, k[:64], v[:64])
    torch.cuda.synchronize()
    assert_codes_equal(c, 0, oracle_q8_heads(k[:64], v[:64], [1, 1], cap=100), [1, 1], 64)
    append_rows(c, 0, k[64:], v[64:])
    torch.cuda.synchronize()
    assert_codes_equal(c, 0, oracle_q8_heads(k, v, [1, 1], cap=100), [1, 1], 100)


def test_q8_all_seqs_append_freezes_each_sequence_at_64():
    say("case: q8_all_seqs")
    r = rng(7)
    B, hkv = 3, 2
    pre = [60, 0, 64]
    c = K.KvCache(K.KIND_Q8, B, hkv, 100)
    src = [channel_rows(r, 80, hkv) for _ in range(B)]
    srcv = [channel_rows(r, 80, hkv) for _ in range(B)]
    for b in range(B):
        append_rows(c, b, src[b][: pre[b]], srcv[b][: pre[b]])
    for t in range(10):
        kt = np.stack([src[b][pre[b] + t] for b in range(B)])
        vt = np.stack([srcv[b][pre[b] + t] for b in range(B)])
        K.kv_append_q8(c, K.ALL_SEQS, 1, dev(kt), dev(vt))
    torch.cuda.synchronize()
    assert list(c.len) == [70, 10, 74] and list(c.frozen) == [1, 0, 1]
    for b in range(B):
        n = pre[b] + 10
        assert_codes_equal(c, b, oracle_q8_heads(src[b][:n], srcv[b][:n], [1, 1], cap=100), [1, 1], n)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def run_decode_case(kind, lens, hkv, hpk, alive, seed, scale_rows=False, opts=None):
    """opts: None, or dict(first=[B] or None, softcap=float, sinks=[Hq] or
    None) for the _ex calls ([P2] attend_group_upto options)."""
    r = rng(seed)
    B = len(lens)
    cap = max(max(lens), 1)
    c = K.KvCache(kind, B, hkv, cap, alive=alive)
    units = [[None] * hkv for _ in range(B)]
    for b, n in enumerate(lens):
        k = channel_rows(r, n, hkv) if scale_rows else r.standard_normal((n, hkv, 128)).astype(np.float32)
        v = channel_rows(r, n, hkv) if scale_rows else r.standard_normal((n, hkv, 128)).astype(np.float32)
        if n:
            append_rows(c, b, k, v)
        if kind == K.KIND_Q8:
            heads = oracle_q8_heads(k, v, alive, cap=cap)
            torch.cuda.synchronize()
            if n:
                assert_codes_equal(c, b, heads, alive, n)
            for g in range(hkv):
                if alive[g] and n:
                    units[b][g] = ("q8", heads[g])
        else:
            for g in range(hkv):
                if alive[g] and n:
                    units[b][g] = ("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g]))
    hq = hkv * hpk
    q = r.standard_normal((B, hq, 128)).astype(np.float32)
    qd = dev(q)
    out = torch.full((B, hq, 128), np.nan, device="cuda")
    if opts is None:
        fn = K.decode_attn_f32 if kind == K.KIND_F32 else K.decode_attn_q8
        call = lambda o: fn(c, hq, qd, o)
        ref_kw = {}
    else:
        fn = K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex
        z = opts.get("sinks")
        zd = None if z is None else dev(np.asarray(z, np.float32))
        o8 = K.DecodeOpts(first=opts.get("first"), softcap=opts.get("softcap", 0.0), sinks=zd)
        call = lambda o: fn(c, hq, qd, o, o8)
        ref_kw = dict(first=opts.get("first"), softcap=opts.get("softcap", 0.0), sinks=z)
    call(out)
    out2 = torch.full_like(out, np.nan)
    call(out2)
    torch.cuda.synchronize()
    got, got2 = host(out), host(out2)
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32)), "decode is not deterministic"
    ref = oracle.decode(q, units, hkv, threads=THREADS, **ref_kw)
    err = max_err(got, ref)
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
    for b in range(B):
        for h in range(hq):
            if not alive[h // hpk] or lens[b] == 0:
                assert not got[b, h].any()
    return c


@pytest.mark.parametrize("hpk", [1, 2, 4, 8])
@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8])
def test_decode_small_shapes(kind, hpk):
    """Several chunks, ragged tails, empty and one-row sequences, a dead group,
    capacity exactly full."""
    say("case: decode_small kind", kind, "hpk", hpk)
    lens = [0, 1, 63, 64, 65, 700, 2500]
    run_decode_case(kind, lens, 4, hpk, np.array([1, 1, 0, 1], np.uint8), seed=10 + hpk + 7 * kind,
                    scale_rows=(kind == K.KIND_Q8))


@pytest.mark.parametrize("variant", ["window", "cap_sinks", "all"])
@pytest.mark.parametrize("hpk", [1, 4, 8])
@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8])
def test_decode_options_small(kind, hpk, variant):
    """[P2] attend_group_upto options through decode_attn_*_ex: visible-row
    starts inside the first tile, on tile edges, at len - 1 and past len
    (clamped), the soft-cap on scaled scores, and per-Q-head sinks, against
    the oracle with the same options."""
    say("case: decode_options kind", kind, "hpk", hpk, "variant", variant)
    lens = [0, 1, 63, 64, 65, 700, 2500]
    first = [0, 5, 10, 63, 64, 650, 100] if variant in ("window", "all") else None
    r = rng(40 + hpk + 3 * kind)
    hq = 4 * hpk
    opts = dict(first=first,
                softcap={"window": 0.0, "cap_sinks": 5.0, "all": 30.0}[variant],
                sinks=None if variant == "window" else (r.standard_normal(hq) * 2).astype(np.float32))
    run_decode_case(kind, lens, 4, hpk, np.array([1, 1, 0, 1], np.uint8), seed=50 + hpk + 7 * kind,
                    scale_rows=(kind == K.KIND_Q8), opts=opts)


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8])
def test_decode_options_none_equal_plain_call(kind):
    """opts = NULL, and options that change nothing (first 0, cap 0, no
    sinks), give the plain call's bits."""
    say("case: decode_options_neutral kind", kind)
    r = rng(60)
    c = K.KvCache(kind, 3, 2, 300)
    lens = [300, 17, 129]
    for b, n in enumerate(lens):
        append_rows(c, b, r.standard_normal((n, 2, 128)).astype(np.float32),
                    r.standard_normal((n, 2, 128)).astype(np.float32))
    q = dev(r.standard_normal((3, 8, 128)).astype(np.float32))
    outs = [torch.full((3, 8, 128), np.nan, device="cuda") for _ in range(3)]
    plain = K.decode_attn_f32 if kind == K.KIND_F32 else K.decode_attn_q8
    ex = K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex
    plain(c, 8, q, outs[0])
    ex(c, 8, q, outs[1], None)
    ex(c, 8, q, outs[2], K.DecodeOpts(first=[0, 0, 0], softcap=0.0))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(host(o).view(np.uint32), host(outs[0]).view(np.uint32))


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8])
def test_decode_batch_over_one_launch(kind):
    """More sequences than one launch's table holds (130 > 128)."""
    say("case: decode_batch_130 kind", kind)
    lens = list(rng(3).integers(0, 90, 130))
    run_decode_case(kind, lens, 2, 2, np.array([1, 1], np.uint8), seed=33 + kind,
                    scale_rows=(kind == K.KIND_Q8))


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8])
def test_decode_all_heads_dead(kind):
    say("case: all_dead kind", kind)
    c = K.KvCache(kind, 2, 2, 16, alive=np.zeros(2, np.uint8))
    fn = K.kv_append_f32 if kind == K.KIND_F32 else K.kv_append_q8
    x = dev(np.ones((5, 2, 128), np.float32))
    fn(c, 0, 5, x, x)
    q = dev(np.ones((2, 4, 128), np.float32))
    out = torch.full((2, 4, 128), np.nan, device="cuda")
    (K.decode_attn_f32 if kind == K.KIND_F32 else K.decode_attn_q8)(c, 4, q, out)
    torch.cuda.synchronize()
    assert list(c.len) == [5, 0] and not host(out).any()


def test_q8_lossless_rows_equal_f32():
    """Integer rows whose groups hold +-127, times 2^-7, quantise losslessly
    (every scale is exactly 2^-7); before the freeze the q8 decode then equals
    the f32 decode of the same values (both within 1e-5 of the oracle)."""
    say("case: q8_lossless")
    r = rng(11)
    n, hkv, hpk = 60, 2, 4
    x = r.integers(-127, 128, (2, n, hkv, 128)).astype(np.float32)
    x[..., ::32] = 127.0
    x *= np.float32(2.0 ** -7)
    k, v = x[0], x[1]
    cf = K.KvCache(K.KIND_F32, 1, hkv, n)
    cq = K.KvCache(K.KIND_Q8, 1, hkv, n)
    append_rows(cf, 0, k, v)
    append_rows(cq, 0, k, v)
    q = (r.standard_normal((1, hkv * hpk, 128)) * 3.0).astype(np.float32)
    of = torch.zeros((1, hkv * hpk, 128), device="cuda")
    oq = torch.zeros_like(of)
    K.decode_attn_f32(cf, hkv * hpk, dev(q), of)
    K.decode_attn_q8(cq, hkv * hpk, dev(q), oq)
    torch.cuda.synchronize()
    assert not cq.frozen[0] and np.all(host(cq.view("ks"))[0, :, :n] == np.float32(2.0 ** -7))
    units = [[("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g])) for g in range(hkv)]]
    ref = oracle.decode(q, units, hkv)
    assert max_err(host(of), ref) <= F32_TOL and max_err(host(oq), ref) <= F32_TOL
    assert np.max(np.abs(host(of) - host(oq))) <= F32_TOL


# ---------------------------------------------------------------------------
# R-SWA
# ---------------------------------------------------------------------------
def rswa_run(nh, prefill, steps, seed, check_every=1, batch=1, hpk=1, kind=K.KIND_F32):
    """Drive rswa_decode for `steps` steps on `batch` streams; compare outputs
    every `check_every` steps and the ring slots at the end.  kind KIND_I8:
    the int8 mirror, compared with the oracle's int8 route and codec."""
    r = rng(seed)
    W = K.RING_WINDOW
    pre = [prefill + 3 * b for b in range(batch)]
    cap = max(pre) + W
    c = K.KvCache(kind, batch, nh, cap)
    rings = K.Rings(batch)
    ref_k = [r.standard_normal((p, nh, 128)).astype(np.float32) for p in pre]
    ref_v = [r.standard_normal((p, nh, 128)).astype(np.float32) for p in pre]
    models = []
    for b in range(batch):
        append_rows(c, b, ref_k[b], ref_v[b])
        K.rswa_record_prefill(c, rings, b)
        m = oracle.RingModel(W)
        m.record_prefill(pre[b])
        models.append(m)
    hq = nh * hpk
    tok_k, tok_v = [], []
    out = torch.zeros((batch, hq, 128), device="cuda")
    for t in range(steps):
        q = r.standard_normal((batch, hq, 128)).astype(np.float32)
        kt = r.standard_normal((batch, nh, 128)).astype(np.float32)
        vt = r.standard_normal((batch, nh, 128)).astype(np.float32)
        tok_k.append(kt)
        tok_v.append(vt)
        K.rswa_decode(c, rings, hq, dev(q), dev(kt), dev(vt), out)
        for b in range(batch):
            models[b].write(t)
            assert rings[b].ring_len == models[b].ring_len and rings[b].ring_pos == models[b].ring_pos
            assert c.len[b] == models[b].effective_len()
        if t % check_every == 0 or t == steps - 1:
            torch.cuda.synchronize()
            got = host(out)
            units = []
            for b in range(batch):
                win = models[b].window()
                kk = np.concatenate([ref_k[b], np.stack([tok_k[s][b] for s in win])])
                vv = np.concatenate([ref_v[b], np.stack([tok_v[s][b] for s in win])])
                if kind == K.KIND_F32:
                    units.append([("f32", np.ascontiguousarray(kk[:, g]), np.ascontiguousarray(vv[:, g]))
                                  for g in range(nh)])
                else:
                    units.append([("i8", i8_head(kk[:, g], vv[:, g])) for g in range(nh)])
            ref = oracle.decode(q, units, nh, threads=THREADS)
            err = max_err(got, ref)
            assert err <= F32_TOL, (t, err)
    torch.cuda.synchronize()
    if kind == K.KIND_I8:
        # every stored row (reference and ring slot) is the page's codec of its source row
        kq, ks, vq, vs = (host(c.view(nm)) for nm in ("kq", "ks", "vq", "vs"))
        for b in range(batch):
            m = models[b]
            for g in range(nh):
                src_k = np.concatenate([ref_k[b][:, g]] + [tok_k[t][b][g][None] for t in m.physical()])
                src_v = np.concatenate([ref_v[b][:, g]] + [tok_v[t][b][g][None] for t in m.physical()])
                h = i8_head(src_k, src_v)
                n = src_k.shape[0]
                assert np.array_equal(kq[b, g, :n], h.kq[:n]) and np.array_equal(vq[b, g, :n], h.vq[:n]), (b, g)
                assert np.array_equal(ks[b, g, :n].view(np.uint32), h.ks[:n].view(np.uint32)), (b, g)
                assert np.array_equal(vs[b, g, :n].view(np.uint32), h.vs[:n].view(np.uint32)), (b, g)
        return rings
    kk, vv = host(c.view("k")), host(c.view("v"))
    for b in range(batch):
        m = models[b]
        # reference block untouched, ring slot of token t is t mod W
        assert np.array_equal(kk[b, :, : pre[b]], ref_k[b].transpose(1, 0, 2))
        assert np.array_equal(vv[b, :, : pre[b]], ref_v[b].transpose(1, 0, 2))
        for s, t in enumerate(m.physical()):
            assert s == t % W
            assert np.array_equal(kk[b, :, pre[b] + s], tok_k[t][b])
            assert np.array_equal(vv[b, :, pre[b] + s], tok_v[t][b])
    return rings


def i8_head(k, v):
    h = oracle.I8Head(cap=max(k.shape[0], 1))
    if k.shape[0]:
        h.append(k, v)
    return h


def test_rswa_i8_small_batched_empty():
    """The int8 mirror through the same R-SWA drives as the f32 cases below:
    ring wrap, three streams with GQA groups, an empty reference block."""
    say("case: rswa i8 small / batched / empty reference")
    rings = rswa_run(nh=4, prefill=5, steps=300, seed=31, check_every=7, kind=K.KIND_I8)
    assert rings[0].ring_len == 128 and rings[0].ring_pos == 300 % 128
    rswa_run(nh=2, prefill=9, steps=140, seed=32, check_every=13, batch=3, hpk=2, kind=K.KIND_I8)
    rswa_run(nh=3, prefill=0, steps=5, seed=33, kind=K.KIND_I8)


def test_rswa_small_wraps_ring():
    say("case: rswa_small")
    rings = rswa_run(nh=4, prefill=5, steps=300, seed=21, check_every=7)
    assert rings[0].ring_len == 128 and rings[0].ring_pos == 300 % 128 and rings[0].writes == 300


def test_rswa_batched_streams_and_gqa():
    say("case: rswa_batched")
    rswa_run(nh=2, prefill=9, steps=140, seed=22, check_every=13, batch=3, hpk=2)


def test_rswa_empty_reference():
    say("case: rswa_empty_reference")
    rswa_run(nh=3, prefill=0, steps=5, seed=23)


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration bench.py times
# ---------------------------------------------------------------------------
def rswa_workload(name, check_steps):
    spec = workloads.get(name)
    W = spec.window
    c = K.KvCache(K.KIND_F32, 1, spec.n_heads, spec.prefill + W)
    rings = K.Rings(1)
    rk, rv = spec.reference()
    append_rows(c, 0, rk.transpose(1, 0, 2), rv.transpose(1, 0, 2))
    K.rswa_record_prefill(c, rings, 0)
    m = oracle.RingModel(W)
    m.record_prefill(spec.prefill)
    out = torch.zeros((1, spec.n_heads, 128), device="cuda")
    toks = {}
    for t in range(spec.writes):
        q, kt, vt = spec.step(t)
        toks[t] = (kt, vt)
        K.rswa_decode(c, rings, spec.n_heads, dev(q[None]), dev(kt[None]), dev(vt[None]), out)
        m.write(t)
        if t in check_steps:
            torch.cuda.synchronize()
            win = m.window()
            units = [[("f32",
                       np.concatenate([rk[g], np.stack([toks[s][0][g] for s in win])]),
                       np.concatenate([rv[g], np.stack([toks[s][1][g] for s in win])]))
                      for g in range(spec.n_heads)]]
            ref = oracle.decode(q[None], units, spec.n_heads, threads=THREADS)
            err = max_err(host(out), ref)
            say("  %s step %d max err %.3g" % (name, t, err))
            assert err <= F32_TOL, (t, err)
    torch.cuda.synchronize()
    assert rings[0].ring_pos == spec.writes % W and rings[0].ring_len == min(spec.writes, W)
    kk = host(c.view("k"))[0]
    assert np.array_equal(kk[:, : spec.prefill], rk)
    for s, t in enumerate(m.physical()):
        assert np.array_equal(kk[:, spec.prefill + s], toks[t][0])


def test_workload_rswa_f32():
    say("case: workload rswa_f32")
    rswa_workload("rswa_f32", check_steps=set(range(165)))


def test_workload_rswa_long_f32():
    say("case: workload rswa_long_f32")
    rswa_workload("rswa_long_f32", check_steps={0, 127, 128, 250, 499})


def gqa_workload(name, sample_units=None, window=None, softcap=0.0, sinks_seed=None):
    """window: rows visible per sequence (first = len - window); softcap and
    seeded per-Q-head sinks go through decode_attn_*_ex when given."""
    from concurrent.futures import ThreadPoolExecutor
    spec = workloads.get(name)
    lens = spec.lengths()
    alive = spec.alive()
    kind = K.KIND_F32 if spec.kind == "f32" else K.KIND_Q8
    c = K.KvCache(kind, spec.batch, spec.n_kv_heads, int(lens.max()), alive=alive)
    units = [[None] * spec.n_kv_heads for _ in range(spec.batch)]

    def gen(b):
        return spec.kv_rows(b)

    with ThreadPoolExecutor(THREADS) as ex:
        for b, (k, v) in enumerate(ex.map(gen, range(spec.batch))):
            append_rows(c, b, k, v)
            if kind == K.KIND_Q8:
                heads = oracle_q8_heads(k, v, alive, cap=int(lens[b]))
                torch.cuda.synchronize()
                assert_codes_equal(c, b, heads, alive, int(lens[b]))
                for g in range(spec.n_kv_heads):
                    if alive[g]:
                        units[b][g] = ("q8", heads[g])
            else:
                for g in range(spec.n_kv_heads):
                    if alive[g]:
                        units[b][g] = ("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g]))
    say("  %s appended %d rows" % (name, int(lens.sum())))
    q = spec.query()
    out = torch.full((spec.batch, spec.n_q_heads, 128), np.nan, device="cuda")
    if window is None and softcap == 0.0 and sinks_seed is None:
        (K.decode_attn_f32 if kind == K.KIND_F32 else K.decode_attn_q8)(c, spec.n_q_heads, dev(q), out)
        ref_kw = {}
    else:
        first = None if window is None else np.maximum(lens.astype(np.int64) - window, 0).astype(np.int32)
        z = None if sinks_seed is None else (rng(sinks_seed).standard_normal(spec.n_q_heads) * 3).astype(np.float32)
        o = K.DecodeOpts(first=first, softcap=softcap, sinks=None if z is None else dev(z))
        (K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex)(c, spec.n_q_heads, dev(q), out, o)
        ref_kw = dict(first=first, softcap=softcap, sinks=z)
    torch.cuda.synchronize()
    got = host(out)
    ref = oracle.decode(q, units, spec.n_kv_heads, threads=THREADS, only=sample_units, **ref_kw)
    hpk = spec.n_q_heads // spec.n_kv_heads
    pairs = sample_units or [(b, g) for b in range(spec.batch) for g in range(spec.n_kv_heads)]
    err = 0.0
    for b, g in pairs:
        sl = slice(g * hpk, (g + 1) * hpk)
        err = max(err, max_err(got[b, sl], ref[b, sl]))
    say("  %s max err %.3g over %d units" % (name, err, len(pairs)))
    assert err <= F32_TOL, err
    for g in np.flatnonzero(alive == 0):
        assert not got[:, g * hpk:(g + 1) * hpk].any()


def test_workload_gqa_f32():
    say("case: workload gqa_f32")
    gqa_workload("gqa_f32")


def test_workload_gqa_q8():
    say("case: workload gqa_q8")
    gqa_workload("gqa_q8")


@pytest.mark.timeout(900)
def test_workload_batched_q8():
    say("case: workload batched_q8")
    gqa_workload("batched_q8")


def test_workload_gqa_f32_options():
    """gqa_f32 with a 1000-row window, soft-cap 20 and sinks."""
    say("case: workload gqa_f32 + options")
    gqa_workload("gqa_f32", window=1000, softcap=20.0, sinks_seed=70)


def test_workload_gqa_q8_options():
    """gqa_q8 with a 4096-row window, soft-cap 50 and sinks."""
    say("case: workload gqa_q8 + options")
    gqa_workload("gqa_q8", window=4096, softcap=50.0, sinks_seed=71)


@pytest.mark.timeout(900)
def test_workload_batched_q8_options():
    """batched_q8 with an 8192-row window (shorter sequences see all rows),
    soft-cap 30 and sinks."""
    say("case: workload batched_q8 + options")
    gqa_workload("batched_q8", window=8192, softcap=30.0, sinks_seed=72)
