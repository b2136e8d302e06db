"""GPU: the per-row int8 route ([P3] quantize_row_i8, decode_attention_int8)
through the C ABI.  Codes and scales bit-exact against the oracle's codec;
decode outputs within 1e-5 of the oracle, whose query codes come from the
same f32 steps."""
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import workloads
from int8_kv_cache_decode_amd import kvq as K
from gpu_cases import F32_TOL, THREADS, append_rows, dev, host, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


def rng(seed):
    return np.random.default_rng(seed)


def assert_i8_codes_equal(c, b, heads, alive, n):
    kq, ks, vq, vs = (host(c.view(nm)[b]) for nm in ("kq", "ks", "vq", "vs"))     # sequence b only
    gl = 0
    for g, live in enumerate(alive):
        if not live:
            continue
        h = heads[g]
        assert np.array_equal(kq[gl, :n], h.kq[:n]) and np.array_equal(vq[gl, :n], h.vq[:n]), (b, g)
        assert np.array_equal(ks[gl, :n].view(np.uint32), h.ks[:n].view(np.uint32)), (b, g)
        assert np.array_equal(vs[gl, :n].view(np.uint32), h.vs[:n].view(np.uint32)), (b, g)
        gl += 1


def test_i8_codec_page_fixtures_and_magnitudes(golden_dir):
    """The page's ties-to-even and division fixtures, a zero row, and rows
    of magnitudes 2^-20 .. 2^20, appended in chunks and one row for all."""
    say("case: i8 codec")
    fx = json.load(open(os.path.join(golden_dir, "int8_row_fixtures.json")))
    r = rng(700)
    n, hkv = 90, 2
    rows = np.zeros((n, hkv, 128), np.float32)
    for p in range(n):
        mag = 2.0 ** ((p % 41) - 20)
        rows[p] = ((r.random((hkv, 128)) * 2 - 1) * mag).astype(np.float32)
    rows[0] = 0
    rows[1, 0, :9] = fx["ties_to_even"]["row_prefix"]
    rows[1, 0, 9:] = 0
    rows[2, 1, :] = 0
    rows[2, 1, :2] = [struct.unpack("<f", struct.pack("<I", int(h, 16)))[0] for h in fx["divides"]["row_prefix_bits"]]
    vrows = rows[::-1].copy()
    c = K.KvCache(K.KIND_I8, 2, hkv, n + 1)
    append_rows(c, 0, rows, vrows, chunks=[1, 2, 50])
    append_rows(c, 1, rows[:40], vrows[:40])
    K.kv_append_i8(c, K.ALL_SEQS, 1, dev(rows[40:42]), dev(vrows[40:42]))
    torch.cuda.synchronize()
    assert list(c.len) == [n + 1, 41]
    for b, (kk, vv) in enumerate(((np.concatenate([rows, rows[40:41]]), np.concatenate([vrows, vrows[40:41]])),
                                  (np.concatenate([rows[:40], rows[41:42]]), np.concatenate([vrows[:40], vrows[41:42]]))
                                  )):
        heads = []
        for g in range(hkv):
            h = oracle.I8Head(cap=kk.shape[0])
            h.append(kk[:, g], vv[:, g])
            heads.append(h)
        assert_i8_codes_equal(c, b, heads, [1, 1], kk.shape[0])
    kq = host(c.view("kq"))
    assert kq[0, 0, 1, :9].tolist() == fx["ties_to_even"]["codes_prefix"]
    assert kq[0, 1, 2, :2].tolist() == fx["divides"]["codes_prefix"]
    assert host(c.view("ks"))[0, 0, 0] == 1.0 and not kq[0, :, 0].any()


@pytest.mark.parametrize("hpk", [1, 2, 4, 8])
def test_i8_decode_small_shapes(hpk):
    """Empty, one-row and ragged sequences, a dead group, several tiles."""
    say("case: i8 decode hpk", hpk)
    r = rng(710 + hpk)
    lens = [0, 1, 63, 64, 65, 700, 2500]
    hkv = 4
    alive = np.array([1, 1, 0, 1], np.uint8)
    c = K.KvCache(K.KIND_I8, len(lens), hkv, max(lens), alive=alive)
    units = [[None] * hkv for _ in lens]
    for b, n in enumerate(lens):
        f = np.exp(r.uniform(np.log(0.25), np.log(8.0), (hkv, 128)))
        k = (r.standard_normal((n, hkv, 128)) * f).astype(np.float32)
        v = (r.standard_normal((n, hkv, 128)) * f).astype(np.float32)
        if n:
            append_rows(c, b, k, v)
            for g in range(hkv):
                if alive[g]:
                    h = oracle.I8Head(cap=n)
                    h.append(k[:, g], v[:, g])
                    units[b][g] = ("i8", h)
    hq = hkv * hpk
    q = (r.standard_normal((len(lens), hq, 128)) * 2).astype(np.float32)
    out, out2 = (torch.full((len(lens), hq, 128), np.nan, device="cuda") for _ in range(2))
    K.decode_attn_i8(c, hq, dev(q), out)
    K.decode_attn_i8(c, hq, dev(q), out2)
    torch.cuda.synchronize()
    got = host(out)
    assert np.array_equal(got.view(np.uint32), host(out2).view(np.uint32))
    ref = oracle.decode(q, units, hkv, threads=THREADS)
    err = max_err(got, ref)
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
    for b in range(len(lens)):
        for h in range(hq):
            if not alive[h // hpk] or lens[b] == 0:
                assert not got[b, h].any()


@pytest.mark.timeout(900)
def test_i8_workload_batched():
    """The batched workload's shapes (64 sequences, 32 Q / 8 KV heads,
    lengths U[1024, 32768], per-channel factors) through the i8 codec."""
    say("case: i8 workload batched")
    from concurrent.futures import ThreadPoolExecutor
    spec = workloads.get("batched_q8")
    lens = spec.lengths()
    c = K.KvCache(K.KIND_I8, spec.batch, spec.n_kv_heads, int(lens.max()))
    units = [[None] * spec.n_kv_heads for _ in range(spec.batch)]

    def build(b):
        k, v = spec.kv_rows(b)
        hs = []
        for g in range(spec.n_kv_heads):
            h = oracle.I8Head(cap=int(lens[b]))
            h.append(k[:, g], v[:, g])
            hs.append(h)
        return k, v, hs

    with ThreadPoolExecutor(THREADS) as ex:
        for b, (k, v, hs) in enumerate(ex.map(build, range(spec.batch))):
            append_rows(c, b, k, v)
            units[b] = [("i8", h) for h in hs]
            # every sequence's codes and row scales, bit for bit
            torch.cuda.synchronize()
            assert_i8_codes_equal(c, b, hs, [1] * spec.n_kv_heads, int(lens[b]))
    q = spec.query()
    out = torch.full((spec.batch, spec.n_q_heads, 128), np.nan, device="cuda")
    K.decode_attn_i8(c, spec.n_q_heads, dev(q), out)
    torch.cuda.synchronize()
    ref = oracle.decode(q, units, spec.n_kv_heads, threads=THREADS)
    err = max_err(host(out), ref)
    say("  i8 batched max err %.3g" % err)
    assert err <= F32_TOL, err


def rswa_i8_workload(name, check_steps):
    """[P3] attention() on the int8 mirror: reference rows appended through
    the int8 codec, then write_decode_step (the step's row quantised into
    its ring slot) + decode_attention_int8 per step.  Outputs against the
    oracle over the reference rows and the live ring in slot order; every
    stored code and scale against the oracle's codec."""
    spec = workloads.get(name)
    W = spec.window
    c = K.KvCache(K.KIND_I8, 1, spec.n_heads, spec.prefill + W)
    rings = K.Rings(1)
    rk, rv = spec.reference()
    append_rows(c, 0, rk.transpose(1, 0, 2), rv.transpose(1, 0, 2))
    K.rswa_record_prefill(c, rings, 0)
    m = oracle.RingModel(W)
    m.record_prefill(spec.prefill)
    out = torch.full((1, spec.n_heads, 128), np.nan, device="cuda")
    toks = {}

    def heads(rows_of):
        hs = []
        for g in range(spec.n_heads):
            kk, vv = rows_of(g)
            h = oracle.I8Head(cap=kk.shape[0])
            h.append(kk, vv)
            hs.append(h)
        return hs

    for t in range(spec.writes):
        q, kt, vt = spec.step(t)
        toks[t] = (kt, vt)
        K.rswa_decode(c, rings, spec.n_heads, dev(q[None]), dev(kt[None]), dev(vt[None]), out)
        m.write(t)
        if t in check_steps:
            torch.cuda.synchronize()
            win = m.window()
            hs = heads(lambda g: (np.concatenate([rk[g], np.stack([toks[s][0][g] for s in win])]),
                                  np.concatenate([rv[g], np.stack([toks[s][1][g] for s in win])])))
            ref = oracle.decode(q[None], [[("i8", h) for h in hs]], spec.n_heads, threads=THREADS)
            err = max_err(host(out), ref)
            say("  %s i8 step %d max err %.3g" % (name, t, err))
            assert err <= F32_TOL, (t, err)
    torch.cuda.synchronize()
    assert rings[0].ring_pos == spec.writes % W and rings[0].ring_len == min(spec.writes, W)
    phys = m.physical()
    hs = heads(lambda g: (np.concatenate([rk[g], np.stack([toks[t][0][g] for t in phys])]),
                          np.concatenate([rv[g], np.stack([toks[t][1][g] for t in phys])])))
    assert_i8_codes_equal(c, 0, hs, [1] * spec.n_heads, spec.prefill + len(phys))


def test_rswa_i8_small():
    say("case: rswa i8 rswa_f32")
    rswa_i8_workload("rswa_f32", check_steps=set(range(0, 165, 3)) | {127, 128, 164})


def test_rswa_i8_long():
    say("case: rswa i8 rswa_long_f32")
    rswa_i8_workload("rswa_long_f32", check_steps={0, 127, 128, 250, 499})
