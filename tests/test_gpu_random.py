"""GPU: seeded random configurations of the decode calls against the oracle.

Each case draws a cache kind (f32, q8 or the per-row int8 kind), a batch
of 1..6 sequences, 1..8 KV heads with a random alive mask, a group size in
{1, 2, 4, 8}, lengths from 0 to a few thousand rows (empty, one-row,
ragged-tail and multi-tile sequences, q8 ones on both sides of the row-64
freeze), rows drawn as the workloads of their kind draw them (f32: unit
normal; q8 and int8: unit normal times per-channel factors log-uniform in
[0.25, 8], as the q8 workloads), and -- for the f32
and q8 kinds -- the [P2] attend_group_upto options (visible-row starts
inside, on and past tile edges and past the length, a soft-cap, sink
logits).  The outputs are compared with the oracle's f64 attention element by
element (q8 and int8: on the oracle's own codec output, whose codes and scales
are checked bit for bit first), and Q heads of dead groups or empty
sequences must be exactly zero."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import F32_TOL, THREADS, append_rows, assert_codes_equal, dev, host, max_err, oracle_q8_heads, say
from int8_kv_cache_decode_amd import kvq as K

pytestmark = pytest.mark.gpu

KINDS = (K.KIND_F32, K.KIND_Q8, K.KIND_I8)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


def draw(seed):
    r = np.random.default_rng(seed)
    kind = KINDS[seed % 3]
    B = int(r.integers(1, 7))
    hkv = int(r.integers(1, 9))
    hpk = int(r.choice([1, 2, 4, 8]))
    alive = (r.random(hkv) < 0.8).astype(np.uint8)
    choices = [0, 1, 15, 16, 17, 63, 64, 65, 200, 1000, 2049, 3001]
    lens = [int(r.choice(choices)) if r.random() < 0.5 else int(r.integers(0, 3200)) for _ in range(B)]
    opts = None
    if kind != K.KIND_I8 and r.random() < 0.6:
        first = [int(r.integers(0, max(n, 1) + 40)) for n in lens] if r.random() < 0.7 else None
        softcap = float(r.choice([0.0, 3.0, 30.0]))
        sinks = (r.standard_normal(hkv * hpk) * 2).astype(np.float32) if r.random() < 0.5 else None
        opts = dict(first=first, softcap=softcap, sinks=sinks)
    return r, kind, lens, hkv, hpk, alive, opts


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_configuration(seed):
    r, kind, lens, hkv, hpk, alive, opts = draw(seed)
    say("case: random seed", seed, "kind", kind, "lens", lens, "hkv", hkv, "hpk", hpk, "alive", alive.tolist(),
        "opts", None if opts is None else {k: (v if not isinstance(v, np.ndarray) else "sinks") for k, v in opts.items()})
    B = len(lens)
    cap = max(max(lens), 1)
    c = K.KvCache(kind, B, hkv, cap, alive=alive)
    units = [[None] * hkv for _ in range(B)]
    # f32 rows unit-scale, as the f32 workloads (scaled f32 rows with queries
    # up to 3x put the f32 scores' rounding at 1.0-1.2e-5 on outputs of
    # magnitude ~20: past an absolute bound fixed for unit-scale f32 rows)
    fac = np.exp(r.uniform(np.log(0.25), np.log(8.0), (2, hkv, 128))).astype(np.float32)
    if kind == K.KIND_F32:
        fac[:] = 1.0
    for b, n in enumerate(lens):
        k = (r.standard_normal((n, hkv, 128)) * fac[0]).astype(np.float32)
        v = (r.standard_normal((n, hkv, 128)) * fac[1]).astype(np.float32)
        if n:
            cuts = sorted(set(int(x) for x in r.integers(1, n, 2))) if n > 2 and r.random() < 0.5 else None
            append_rows(c, b, k, v, chunks=cuts)
        if kind == K.KIND_Q8:
            heads = oracle_q8_heads(k, v, alive, cap=cap)
            torch.cuda.synchronize()
            if n:
                assert_codes_equal(c, b, heads, alive, n)
            for g in range(hkv):
                if alive[g] and n:
                    units[b][g] = ("q8", heads[g])
        elif kind == K.KIND_I8:
            for g in range(hkv):
                if alive[g] and n:
                    h = oracle.I8Head(cap=cap)
                    h.append(k[:, g], v[:, g])
                    units[b][g] = ("i8", h)
        else:
            for g in range(hkv):
                if alive[g] and n:
                    units[b][g] = ("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g]))
    if kind == K.KIND_I8:
        torch.cuda.synchronize()
        kq, ks = host(c.view("kq")), host(c.view("ks"))
        vq, vs = host(c.view("vq")), host(c.view("vs"))
        for b, n in enumerate(lens):
            slot = 0
            for g in range(hkv):
                if not alive[g]:
                    continue
                if n:
                    h = units[b][g][1]
                    assert np.array_equal(kq[b, slot, :n], h.kq[:n]), ("kq", b, g)
                    assert np.array_equal(ks[b, slot, :n].view(np.uint32), h.ks[:n].view(np.uint32)), ("ks", b, g)
                    assert np.array_equal(vq[b, slot, :n], h.vq[:n]), ("vq", b, g)
                    assert np.array_equal(vs[b, slot, :n].view(np.uint32), h.vs[:n].view(np.uint32)), ("vs", b, g)
                slot += 1
    hq = hkv * hpk
    q = (r.standard_normal((B, hq, 128)) * r.uniform(0.5, 3.0)).astype(np.float32)
    out = torch.full((B, hq, 128), float("nan"), device="cuda")
    ref_kw = {}
    if opts is None:
        {K.KIND_F32: K.decode_attn_f32, K.KIND_Q8: K.decode_attn_q8, K.KIND_I8: K.decode_attn_i8}[kind](
            c, hq, dev(q), out)
    else:
        z = opts["sinks"]
        o8 = K.DecodeOpts(first=opts["first"], softcap=opts["softcap"], sinks=None if z is None else dev(z))
        (K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex)(c, hq, dev(q), out, o8)
        ref_kw = dict(first=opts["first"], softcap=opts["softcap"], sinks=z)
    torch.cuda.synchronize()
    got = host(out)
    ref = oracle.decode(q, units, hkv, threads=THREADS, **ref_kw)
    err = max_err(got, ref)
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
    for b in range(B):
        for h in range(hq):
            if not alive[h // hpk] or lens[b] == 0:
                assert not got[b, h].any(), (b, h)
