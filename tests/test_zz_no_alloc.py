"""GPU: decode_attn_q8_noalloc, the variant of decode_attn_q8 whose partial
softmax states live in the library's static device array, through the C
ABI.  Two calls in a row -- the second on a smaller cache, after the first
left its partials in the array -- each equal, bit for bit, to
decode_attn_q8 with a caller's workspace on the same cache, and within the
f32 tolerance of the oracle's decode."""
import numpy as np
import pytest
import torch

import oracle
from int8_kv_cache_decode_amd import kvq as K
from gpu_cases import F32_TOL, THREADS, append_rows, dev, host, max_err, oracle_q8_heads, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


def build_case(seed, lens, hkv, hpk, alive):
    r = np.random.default_rng(seed)
    cap = max(lens)
    c = K.KvCache(K.KIND_Q8, len(lens), hkv, cap, alive=alive)
    units = []
    for b, n in enumerate(lens):
        f = np.exp(r.uniform(np.log(0.25), np.log(8.0), (hkv, 128)))
        k = (r.standard_normal((n, hkv, 128)) * f).astype(np.float32)
        v = (r.standard_normal((n, hkv, 128)) * f[::-1]).astype(np.float32)
        append_rows(c, b, k, v)
        heads = oracle_q8_heads(k, v, alive, cap=n)
        units.append([("q8", heads[g]) if alive[g] and n else None for g in range(hkv)])
    q = r.standard_normal((len(lens), hkv * hpk, 128)).astype(np.float32)
    return c, q, units


def test_noalloc_decode_twice_second_smaller():
    cases = [
        # 5 sequences (lengths across the freeze, one empty), 4 KV heads with
        # a dead group, group 4: several tiles per segment and a ragged tail
        (7100, [300, 1, 0, 2000, 65], 4, 4, np.array([1, 1, 0, 1], np.uint8)),
        # then a smaller cache: 2 sequences, 2 KV heads, group 2
        (7101, [100, 20], 2, 2, np.array([1, 1], np.uint8)),
    ]
    for seed, lens, hkv, hpk, alive in cases:
        say("case: noalloc q8 decode lens", lens, "hkv", hkv, "hpk", hpk)
        c, qh, units = build_case(seed, lens, hkv, hpk, alive)
        hq = hkv * hpk
        q = dev(qh)
        want = torch.full((len(lens), hq, 128), np.nan, device="cuda")
        got = torch.full((len(lens), hq, 128), np.nan, device="cuda")
        K.decode_attn_q8(c, hq, q, want)
        K.decode_attn_q8_noalloc(c, hq, q, got)
        torch.cuda.synchronize()
        g, w = host(got), host(want)
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), np.abs(g - w).max()
        err = max_err(g, oracle.decode(qh, units, hkv, threads=THREADS))
        say("  max err vs oracle %.3g" % err)
        assert err <= F32_TOL, err


def test_noalloc_decode_replays_from_a_graph():
    """The callers this entry point is for include code under HIP graph
    capture: a captured call is replayed four times, each time after an eager
    call of the same entry point on another cache has overwritten the static
    array, and every replay equals decode_attn_q8 with a caller's workspace
    bit for bit."""
    say("case: noalloc q8 decode captured in a graph")
    c, qh, _ = build_case(7200, [900, 33, 0, 64], 3, 4, np.array([1, 0, 1], np.uint8))
    other, qo_h, _ = build_case(7201, [2500, 1200], 2, 8, np.array([1, 1], np.uint8))
    hq, hq_o = 3 * 4, 2 * 8
    q, qo = dev(qh), dev(qo_h)
    want_t = torch.full((4, hq, 128), np.nan, device="cuda")
    K.decode_attn_q8(c, hq, q, want_t)
    out = torch.full((4, hq, 128), np.nan, device="cuda")
    out_o = torch.empty((2, hq_o, 128), device="cuda")
    K.decode_attn_q8_noalloc(c, hq, q, out)          # eager first: the device address lookup happens here
    torch.cuda.synchronize()
    want = host(want_t).copy()
    assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.decode_attn_q8_noalloc(c, hq, q, out)
    for i in range(4):
        K.decode_attn_q8_noalloc(other, hq_o, qo, out_o)   # another call leaves its partials in the array
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32)), i
    assert not host(out)[2].any()                    # the empty sequence
