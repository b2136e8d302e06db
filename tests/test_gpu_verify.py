"""GPU: K-token R-SWA verify ([P3] verify_attention) through the C ABI
against the oracle's definition (the i-th of K sequential decode steps),
in warm-up, crossing the ring window and in steady state; the cache and the
ring cursors must be left exactly as they were."""
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


BUFS = {K.KIND_F32: ("k", "v"), K.KIND_I8: ("kq", "ks", "vq", "vs")}


def run_verify(batch, hkv, hpk, prefill, n_hist, n_draft, seed, kind=K.KIND_F32, spread=False):
    """spread: every key row is 0 on channel 0 except one reference spike row
    per (sequence, KV head) at 64, and each query is +-32 on channel 0 (sign
    alternating over the queries of a KV head) and 0 elsewhere: the spike
    scores +-181 (natural units), every other row exactly 0, so a running max
    taken over another query's lanes, or missing the spike's lane, gives 0/0
    or inf (see tests/test_gpu_spread.py)."""
    r = rng(seed)
    W = K.RING_WINDOW
    c = K.KvCache(kind, batch, hkv, prefill + W)
    rings = K.Rings(batch)
    hq = hkv * hpk
    ref = [(r.standard_normal((prefill, hkv, 128)).astype(np.float32),
            r.standard_normal((prefill, hkv, 128)).astype(np.float32)) for _ in range(batch)]
    if spread:
        for b in range(batch):
            ref[b][0][:, :, 0] = 0.0
            for g in range(hkv):
                ref[b][0][(7 + 13 * b + 5 * g) % prefill, g, 0] = 64.0
    for b in range(batch):
        if prefill:
            append_rows(c, b, *ref[b])
        K.rswa_record_prefill(c, rings, b)
    hist_k = r.standard_normal((n_hist, batch, hkv, 128)).astype(np.float32)
    hist_v = r.standard_normal((n_hist, batch, hkv, 128)).astype(np.float32)
    if spread:
        hist_k[..., 0] = 0.0
    out1 = torch.zeros((batch, hq, 128), device="cuda")
    q1 = dev(r.standard_normal((batch, hq, 128)).astype(np.float32))
    for t in range(n_hist):
        K.rswa_decode(c, rings, hq, q1, dev(hist_k[t]), dev(hist_v[t]), out1)
    torch.cuda.synchronize()
    before = ([host(c.view(nm)).copy() for nm in BUFS[kind]], bytes(rings.arr), c.len.copy())
    q = r.standard_normal((batch, n_draft, hq, 128)).astype(np.float32)
    dk = r.standard_normal((batch, n_draft, hkv, 128)).astype(np.float32)
    dv = r.standard_normal((batch, n_draft, hkv, 128)).astype(np.float32)
    if spread:
        dk[..., 0] = 0.0
        q[:] = 0.0
        q[..., 0] = np.where((np.arange(n_draft)[:, None] * hq + np.arange(hq)[None, :]) % 2 == 0, 32.0, -32.0)
    out = torch.full((batch, n_draft, hq, 128), np.nan, device="cuda")
    K.rswa_verify(c, rings, hq, n_draft, dev(q), dev(dk), dev(dv), out)
    out2 = torch.full_like(out, np.nan)
    K.rswa_verify(c, rings, hq, n_draft, dev(q), dev(dk), dev(dv), out2)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all()
    assert np.array_equal(got.view(np.uint32), host(out2).view(np.uint32)), "verify is not deterministic"
    for nm, b0 in zip(BUFS[kind], before[0]):
        assert np.array_equal(host(c.view(nm)).view(np.uint8), b0.view(np.uint8)), nm
    assert bytes(rings.arr) == before[1] and np.array_equal(c.len, before[2])
    err = 0.0
    for b in range(batch):
        ref_k = np.ascontiguousarray(ref[b][0].transpose(1, 0, 2))
        ref_v = np.ascontiguousarray(ref[b][1].transpose(1, 0, 2))
        hk = np.ascontiguousarray(hist_k[:, b].transpose(1, 0, 2))
        hv = np.ascontiguousarray(hist_v[:, b].transpose(1, 0, 2))
        want = oracle.rswa_verify(q[b], ref_k, ref_v, hk, hv, dk[b], dv[b], W,
                                  kind="i8" if kind == K.KIND_I8 else "f32")
        err = max(err, max_err(got[b], want))
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
@pytest.mark.parametrize("hkv,hpk,prefill,n_hist,n_draft", [
    (2, 1, 7, 5, 4),        # warm-up
    (2, 1, 300, 126, 5),    # the drafts fill the ring and evict
    (3, 2, 40, 300, 8),     # steady state, 16 queries per KV head
    (1, 1, 0, 0, 3),        # empty reference, empty ring
    (2, 1, 65, 128, 16),    # ring exactly full, 16 drafts
    (2, 4, 33, 70, 2),      # GQA groups of 4
])
def test_verify_matches_sequential_definition(hkv, hpk, prefill, n_hist, n_draft, kind):
    say("case: verify kind", kind, "hkv", hkv, "hpk", hpk, "prefill", prefill, "hist", n_hist, "drafts", n_draft)
    run_verify(2, hkv, hpk, prefill, n_hist, n_draft, seed=500 + prefill + n_hist + n_draft, kind=kind)


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
@pytest.mark.parametrize("hkv,hpk,n_hist,n_draft", [(2, 1, 20, 8), (2, 4, 130, 4), (1, 2, 127, 7)])
def test_verify_extreme_score_spread(hkv, hpk, n_hist, n_draft, kind):
    say("case: verify spread kind", kind, "hkv", hkv, "hpk", hpk, "hist", n_hist, "drafts", n_draft)
    run_verify(2, hkv, hpk, 300, n_hist, n_draft, seed=800 + n_hist + n_draft, kind=kind, spread=True)


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
def test_verify_long_reference(kind):
    """rswa_long_f32's shape: 10 heads, 32640 reference rows, ring full
    after 500 writes, 8 drafts."""
    say("case: verify long reference kind", kind)
    spec = workloads.get("rswa_long_f32")
    r = rng(600)
    W = spec.window
    c = K.KvCache(kind, 1, spec.n_heads, spec.prefill + W)
    rings = K.Rings(1)
    rk, rv = spec.reference()
    append_rows(c, 0, rk.transpose(1, 0, 2), rv.transpose(1, 0, 2))
    K.rswa_record_prefill(c, rings, 0)
    out1 = torch.zeros((1, spec.n_heads, 128), device="cuda")
    steps = [spec.step(t) for t in range(spec.writes)]
    for qs, ks, vs in steps:
        K.rswa_decode(c, rings, spec.n_heads, dev(qs[None]), dev(ks[None]), dev(vs[None]), out1)
    n_draft = 8
    q = r.standard_normal((1, n_draft, spec.n_heads, 128)).astype(np.float32)
    dk = r.standard_normal((1, n_draft, spec.n_heads, 128)).astype(np.float32)
    dv = r.standard_normal((1, n_draft, spec.n_heads, 128)).astype(np.float32)
    out = torch.full((1, n_draft, spec.n_heads, 128), np.nan, device="cuda")
    K.rswa_verify(c, rings, spec.n_heads, n_draft, dev(q), dev(dk), dev(dv), out)
    torch.cuda.synchronize()
    hk = np.stack([s[1] for s in steps], axis=1)
    hv = np.stack([s[2] for s in steps], axis=1)
    want = oracle.rswa_verify(q[0], rk, rv, hk, hv, dk[0], dv[0], W, kind="i8" if kind == K.KIND_I8 else "f32")
    err = max_err(host(out)[0], want)
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err
