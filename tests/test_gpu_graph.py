"""GPU: the decode calls are safe to capture in a HIP graph -- they enqueue
kernels only (no allocation, no synchronisation, no memset) on the caller's
stream.  A captured call is replayed several times, with eager work and
synchronisations in between, and every replay must equal the eager call bit
for bit.  Calls that move host cursors (appends, rswa_decode) are not
replayable by nature and are not captured."""
import numpy as np
import pytest
import torch

from int8_kv_cache_decode_amd import kvq as K
from gpu_cases import append_rows, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()


def replay_equals_eager(call, out, replays=4):
    call()                                          # eager, also fills the library's per-device caches
    torch.cuda.synchronize()
    want = host(out).copy()
    g = torch.cuda.CUDAGraph()
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for i in range(replays):
        out.fill_(float("nan"))
        noise = torch.randn(1 << 20, device="cuda") * 3.0 + i    # eager work between replays
        noise.sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32)), i
    return want


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_decode_replays_from_a_graph(kind):
    say("case: graph decode kind", kind)
    r = np.random.default_rng(990 + kind)
    lens, hkv, hpk = [700, 0, 2100], 2, 4
    c = K.KvCache(kind, len(lens), hkv, max(lens))
    for b, n in enumerate(lens):
        if n:
            append_rows(c, b, r.standard_normal((n, hkv, 128)).astype(np.float32),
                        r.standard_normal((n, hkv, 128)).astype(np.float32))
    hq = hkv * hpk
    q = dev(r.standard_normal((len(lens), hq, 128)).astype(np.float32))
    out = torch.zeros((len(lens), hq, 128), device="cuda")
    ws = c.workspace(hq)
    fn = {K.KIND_F32: K.decode_attn_f32, K.KIND_Q8: K.decode_attn_q8, K.KIND_I8: K.decode_attn_i8}[kind]
    got = replay_equals_eager(lambda: fn(c, hq, q, out, ws), out)
    assert np.isfinite(got).all() and not got[1].any()
    if kind != K.KIND_I8:
        ex = K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex
        sinks = dev(np.linspace(-2, 2, hq).astype(np.float32))
        o = K.DecodeOpts(first=np.array([600, 0, 5], np.int32), softcap=20.0, sinks=sinks)
        replay_equals_eager(lambda: ex(c, hq, q, out, o, ws), out)


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
def test_verify_replays_from_a_graph(kind):
    """rswa_verify writes nothing, so a captured verify is replayable (the
    int8 kind's draft quantisation into the workspace included)."""
    say("case: graph verify kind", kind)
    r = np.random.default_rng(995 + kind)
    hkv, hpk, pre, n_draft = 2, 2, 300, 4
    c = K.KvCache(kind, 1, hkv, pre + K.RING_WINDOW)
    rings = K.Rings(1)
    append_rows(c, 0, r.standard_normal((pre, hkv, 128)).astype(np.float32),
                r.standard_normal((pre, hkv, 128)).astype(np.float32))
    K.rswa_record_prefill(c, rings, 0)
    hq = hkv * hpk
    o1 = torch.zeros((1, hq, 128), device="cuda")
    for t in range(40):
        K.rswa_decode(c, rings, hq, dev(r.standard_normal((1, hq, 128)).astype(np.float32)),
                      dev(r.standard_normal((1, hkv, 128)).astype(np.float32)),
                      dev(r.standard_normal((1, hkv, 128)).astype(np.float32)), o1)
    q = dev(r.standard_normal((1, n_draft, hq, 128)).astype(np.float32))
    dk = dev(r.standard_normal((1, n_draft, hkv, 128)).astype(np.float32))
    dv = dev(r.standard_normal((1, n_draft, hkv, 128)).astype(np.float32))
    out = torch.zeros((1, n_draft, hq, 128), device="cuda")
    ws = torch.empty(K.kvq_verify_workspace_bytes(c, hq, n_draft), dtype=torch.uint8, device="cuda")
    got = replay_equals_eager(lambda: K.rswa_verify(c, rings, hq, n_draft, q, dk, dv, out, ws), out)
    assert np.isfinite(got).all()
