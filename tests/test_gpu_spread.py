"""GPU parity with extreme score spreads: the tile maxima of the online
softmax must be the true maxima of each Q head.

The online fold of [P3] (fold: rescale by exp(old max - new max)) gives the
same result for any running max that keeps the exponentials finite, so
ordinary inputs cannot tell a correct tile max from one that mixes Q heads
or misses rows.  Here every (sequence, KV head) holds one spike row whose
key is 64 on channel 0; every other row is 0 on channel 0.  The query of Q
head h is +-32 on channel 0 (sign alternating with h) and 0 elsewhere, so
the spike scores +-2048/sqrt(128) = +-181 (natural units) and every other
row scores exactly 0.  A max taken over the wrong head turns a head's
weights into exp(-181) = 0 in f32 (a 0/0 result); a max that misses the
spike's lane turns its weight into exp(+181) = inf.  With the true max the
result is one-hot on the spike's value row (positive heads) or the mean of
the other rows' values (negative heads), within 1e-5 of the float64 oracle.
Spike rows sit at many positions within their 16-row tiles.
"""
import numpy as np
import pytest
import torch

import oracle
from int8_kv_cache_decode_amd import kvq as K
from gpu_cases import F32_TOL, THREADS, append_rows, assert_codes_equal, dev, host, max_err, oracle_q8_heads, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


@pytest.mark.parametrize("hpk", [1, 4, 8])
@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_decode_extreme_score_spread(kind, hpk):
    say("case: score_spread kind", kind, "hpk", hpk)
    r = np.random.default_rng(900 + 10 * kind + hpk)
    lens = [40, 300, 1000]
    hkv, B = 2, 3
    hq = hkv * hpk
    c = K.KvCache(kind, B, hkv, max(lens))
    alive = np.ones(hkv, np.uint8)
    units = [[None] * hkv for _ in range(B)]
    spikes = []
    for b, n in enumerate(lens):
        k = r.standard_normal((n, hkv, 128)).astype(np.float32)
        v = r.standard_normal((n, hkv, 128)).astype(np.float32)
        k[:, :, 0] = 0.0
        for g in range(hkv):
            p = (11 * (b * hkv + g) + 5 + 16 * g) % n
            k[p, g, 0] = 64.0
            spikes.append(p % 16)
        append_rows(c, b, k, v)
        if kind == K.KIND_Q8:
            heads = oracle_q8_heads(k, v, alive, cap=max(lens))
            torch.cuda.synchronize()
            assert_codes_equal(c, b, heads, alive, n)
            units[b] = [("q8", h) for h in heads]
        elif kind == K.KIND_I8:
            for g in range(hkv):
                h = oracle.I8Head(cap=n)
                h.append(k[:, g], v[:, g])
                units[b][g] = ("i8", h)
        else:
            units[b] = [("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g])) for g in range(hkv)]
    assert len(set(spikes)) == len(spikes)          # distinct positions within their tiles
    q = np.zeros((B, hq, 128), np.float32)
    q[:, :, 0] = np.where(np.arange(hq) % 2 == 0, 32.0, -32.0)
    fn = {K.KIND_F32: K.decode_attn_f32, K.KIND_Q8: K.decode_attn_q8, K.KIND_I8: K.decode_attn_i8}[kind]
    out = torch.full((B, hq, 128), np.nan, device="cuda")
    fn(c, hq, dev(q), out)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all()
    ref = oracle.decode(q, units, hkv, threads=THREADS)
    err = max_err(got, ref)
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
