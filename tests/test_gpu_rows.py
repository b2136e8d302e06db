"""GPU: row management around the decode ([P2] LayerKvCache::truncate_last,
trim_window_anchored; [P3] RingCache::checkpoint / rollback_to) through the
C ABI.  Moved rows, codes and scales are compared bit for bit with the rows
they came from; decodes after a trim, a truncate or a rollback are compared
with the oracle over the rows the pages say stay visible, or bit for bit
with a control cache that never took the detour, and with the oracle's
stores / ring model taken through the same truncate or rollback."""
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


def rng(seed):
    return np.random.default_rng(seed)


BUFS = {K.KIND_F32: ("k", "v"), K.KIND_Q8: ("kq", "ks", "vq", "vs"), K.KIND_I8: ("kq", "ks", "vq", "vs")}
DECODE = {K.KIND_F32: K.decode_attn_f32, K.KIND_Q8: K.decode_attn_q8, K.KIND_I8: K.decode_attn_i8}


# (lens, w, slack, align, anchor): overlapping moves (keep > d), disjoint
# ones (keep <= d), many chunks, an anchored cut, and a no-op.
TRIMS = [([3000, 2001], 1400, 150, 16, -1),
         ([2001, 700], 1000, 0, 4, -1),
         ([900, 2500], 300, 2, 64, -1),
         ([1500, 1500], 200, 10, 8, 900),
         ([300, 100], 200, 10, 8, -1),
         # several sequences moving 1 to 10 rounds of rows in the same launches
         ([3000, 2001, 620, 700, 610, 5], 300, 250, 8, -1)]


@pytest.mark.parametrize("all_seqs", [False, True])
@pytest.mark.parametrize("case", range(len(TRIMS)))
@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_trim_window_moves_rows_and_keeps_the_window(kind, case, all_seqs):
    lens, w, slack, align, anchor = TRIMS[case]
    say("case: trim kind", kind, "lens", lens, "w", w, "slack", slack, "align", align, "anchor", anchor,
        "all sequences" if all_seqs else "one call per sequence")
    r = rng(100 + case + 10 * kind)
    hkv, hpk = 3, 2
    alive = np.array([1, 0, 1], np.uint8)
    cap = max(lens)
    c = K.KvCache(kind, len(lens), hkv, cap, alive=alive)
    rows = []
    for b, n in enumerate(lens):
        k = (r.standard_normal((n, hkv, 128)) * 2).astype(np.float32)
        v = (r.standard_normal((n, hkv, 128)) * 2).astype(np.float32)
        append_rows(c, b, k, v)
        rows.append((k, v))
    torch.cuda.synchronize()
    before = {nm: host(c.view(nm)).copy() for nm in BUFS[kind]}
    q = r.standard_normal((len(lens), hkv * hpk, 128)).astype(np.float32)
    want = [oracle.trim_window(0, n, w, slack, align, None if anchor < 0 else anchor,
                               q8_unfrozen=(kind == K.KIND_Q8 and n < 64)) for n in lens]
    if all_seqs:
        nb, nd = K.kv_trim_window(c, K.ALL_SEQS, [0] * len(lens), w, slack, align, anchor)
        assert list(nd) == want and list(nb) == want
        bases = [int(x) for x in nb]
    else:
        bases = []
        for b, n in enumerate(lens):
            base, d = K.kv_trim_window(c, b, 0, w, slack, align, anchor)
            assert d == want[b] and base == d
            bases.append(base)
    assert all(c.len[b] == n - want[b] for b, n in enumerate(lens))
    torch.cuda.synchronize()
    # every live head's rows [d, n) now sit at [0, n - d), bit for bit
    for nm in BUFS[kind]:
        after = host(c.view(nm))
        for b, n in enumerate(lens):
            d = bases[b]
            assert np.array_equal(after[b, :, : n - d].view(np.uint8), before[nm][b, :, d:n].view(np.uint8)), (nm, b)
    if kind == K.KIND_I8:
        # per-row codes do not depend on the other rows: the trimmed cache
        # decodes as a cache that only ever held rows [d, n)
        out = torch.full((len(lens), hkv * hpk, 128), np.nan, device="cuda")
        K.decode_attn_i8(c, hkv * hpk, dev(q), out)
        torch.cuda.synchronize()
        units = [[None] * hkv for _ in lens]
        for b, n in enumerate(lens):
            k, v = rows[b]
            for g in range(hkv):
                if alive[g]:
                    h = oracle.I8Head(cap=n)
                    h.append(k[bases[b]:, g], v[bases[b]:, g])
                    units[b][g] = ("i8", h)
        err = max_err(host(out), oracle.decode(q, units, hkv, threads=THREADS))
        say("  i8 max err %.3g" % err)
        assert err <= F32_TOL, err
        return
    # the windowed decode (first = len - w) of the trimmed cache sees the rows
    # the untrimmed cache's window sees
    first = np.maximum(c.len.astype(np.int64) - w, 0).astype(np.int32)
    out = torch.full((len(lens), hkv * hpk, 128), np.nan, device="cuda")
    fn = K.decode_attn_f32_ex if kind == K.KIND_F32 else K.decode_attn_q8_ex
    fn(c, hkv * hpk, dev(q), out, K.DecodeOpts(first=first))
    torch.cuda.synchronize()
    units = [[None] * hkv for _ in lens]
    full_first = []
    for b, n in enumerate(lens):
        k, v = rows[b]
        full_first.append(max(n - w, 0))
        if kind == K.KIND_Q8:
            heads = oracle_q8_heads(k, v, alive, cap=n)
            for g in range(hkv):
                units[b][g] = ("q8", heads[g]) if alive[g] else None
        else:
            for g in range(hkv):
                units[b][g] = ("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g])) if alive[g] else None
    ref = oracle.decode(q, units, hkv, threads=THREADS, first=full_first)
    err = max_err(host(out), ref)
    say("  max err %.3g" % err)
    assert err <= F32_TOL, err


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_Q8, K.KIND_I8])
def test_truncate_then_append_equals_never_appended(kind):
    """[P2] truncate_last after a speculative append: the replacement rows
    land where the rejected ones were; storage and decode equal a cache that
    only ever saw the accepted rows (a q8 field frozen before keeps its
    values)."""
    say("case: truncate kind", kind)
    r = rng(200 + kind)
    hkv, hpk, n0 = 2, 4, 150
    base_k = (r.standard_normal((n0, hkv, 128)) * 2).astype(np.float32)
    base_v = (r.standard_normal((n0, hkv, 128)) * 2).astype(np.float32)
    draft = [(r.standard_normal((5, hkv, 128)) * 2).astype(np.float32) for _ in range(2)]
    final = [(r.standard_normal((3, hkv, 128)) * 2).astype(np.float32) for _ in range(2)]
    test = K.KvCache(kind, 1, hkv, 200)
    ctrl = K.KvCache(kind, 1, hkv, 200)
    for cc in (test, ctrl):
        append_rows(cc, 0, base_k, base_v)
    append_rows(test, 0, *draft)
    K.kv_truncate_last(test, 0, 5)
    assert test.len[0] == n0
    for cc in (test, ctrl):
        append_rows(cc, 0, *final)
    torch.cuda.synchronize()
    n = n0 + 3
    for nm in BUFS[kind]:
        a, b = host(test.view(nm)), host(ctrl.view(nm))
        assert np.array_equal(a[:, :, :n].view(np.uint8), b[:, :, :n].view(np.uint8)), nm
    qh = r.standard_normal((1, hkv * hpk, 128)).astype(np.float32)
    q = dev(qh)
    o1, o2 = (torch.full((1, hkv * hpk, 128), np.nan, device="cuda") for _ in range(2))
    fn = DECODE[kind]
    fn(test, hkv * hpk, q, o1)
    fn(ctrl, hkv * hpk, q, o2)
    torch.cuda.synchronize()
    assert np.array_equal(host(o1).view(np.uint32), host(o2).view(np.uint32))
    # against the oracle: its stores take the same appends and the page's
    # truncate (q8: the rejected rows were quantised against the frozen
    # field, which stays), then decode by definition
    units = [[None] * hkv]
    for g in range(hkv):
        if kind == K.KIND_F32:
            units[0][g] = ("f32", np.concatenate([base_k[:, g], final[0][:, g]]),
                           np.concatenate([base_v[:, g], final[1][:, g]]))
            continue
        h = oracle.Q8Head(cap=200) if kind == K.KIND_Q8 else oracle.I8Head(cap=200)
        h.append(base_k[:, g], base_v[:, g])
        h.append(draft[0][:, g], draft[1][:, g])
        h.truncate_last(5)
        h.append(final[0][:, g], final[1][:, g])
        assert h.n == n
        units[0][g] = ("q8" if kind == K.KIND_Q8 else "i8", h)
    if kind == K.KIND_Q8:
        assert_codes_equal(test, 0, [u[1] for u in units[0]], [1] * hkv, n)
    elif kind == K.KIND_I8:
        kq, ks = host(test.view("kq"))[0], host(test.view("ks"))[0]
        for g in range(hkv):
            assert np.array_equal(kq[g, :n], units[0][g][1].kq[:n])
            assert np.array_equal(ks[g, :n].view(np.uint32), units[0][g][1].ks[:n].view(np.uint32))
    err = max_err(host(o1), oracle.decode(qh, units, hkv, threads=THREADS))
    say("  truncate kind %d max err %.3g" % (kind, err))
    assert err <= F32_TOL, err


@pytest.mark.parametrize("kind", [K.KIND_F32, K.KIND_I8])
def test_rswa_rollback_restores_the_accepted_path(kind):
    """[P3] test checkpoint_rollback_restores_ring_rows_byte_identical at the
    decode level: 5 reference rows, 9 accepted steps, checkpoint, 6 draft
    steps, rollback, then more accepted steps: every output and every live
    row equals a control cache that never speculated, and the first dead
    slot still holds a draft row."""
    say("case: rswa rollback kind", kind)
    r = rng(300)
    nh, pf = 4, 5
    test = K.KvCache(kind, 1, nh, pf + 128)
    ctrl = K.KvCache(kind, 1, nh, pf + 128)
    rt, rc = K.Rings(1), K.Rings(1)
    ref = (r.standard_normal((2, pf, nh, 128))).astype(np.float32)
    for cc, rr in ((test, rt), (ctrl, rc)):
        append_rows(cc, 0, ref[0], ref[1])
        K.rswa_record_prefill(cc, rr, 0)
    acc_h = [tuple(r.standard_normal((1, nh, 128)).astype(np.float32) for _ in range(3)) for _ in range(14)]
    drafts_h = [tuple(r.standard_normal((1, nh, 128)).astype(np.float32) + 3 for _ in range(3)) for _ in range(6)]
    acc = [tuple(dev(x) for x in a) for a in acc_h]
    drafts = [tuple(dev(x) for x in d) for d in drafts_h]
    ot, oc = (torch.zeros((1, nh, 128), device="cuda") for _ in range(2))
    # the oracle's ring model takes the same writes, checkpoint and rollback
    model = oracle.RingModel(K.RING_WINDOW)
    model.record_prefill(pf)
    rows = {}

    def oracle_out(q):
        win = model.window()
        kk = np.concatenate([ref[0], np.stack([rows[u][0] for u in win])])
        vv = np.concatenate([ref[1], np.stack([rows[u][1] for u in win])])
        if kind == K.KIND_F32:
            units = [[("f32", np.ascontiguousarray(kk[:, g]), np.ascontiguousarray(vv[:, g])) for g in range(nh)]]
        else:
            units = [[]]
            for g in range(nh):
                h = oracle.I8Head(cap=kk.shape[0])
                h.append(kk[:, g], vv[:, g])
                units[0].append(("i8", h))
        return oracle.decode(q, units, nh, threads=THREADS)

    for t in range(9):
        q, k, v = acc[t]
        K.rswa_decode(test, rt, nh, q, k, v, ot)
        K.rswa_decode(ctrl, rc, nh, q, k, v, oc)
        rows[("a", t)] = (acc_h[t][1][0], acc_h[t][2][0])
        model.write(("a", t))
    cp = K.rswa_checkpoint(test, rt, 0)
    mcp = model.checkpoint()
    assert (cp.ring_len, cp.ring_pos, cp.prefill_len) == (9, 9, pf)
    for i, (q, k, v) in enumerate(drafts):
        K.rswa_decode(test, rt, nh, q, k, v, ot)
        rows[("d", i)] = (drafts_h[i][1][0], drafts_h[i][2][0])
        model.write(("d", i))
    torch.cuda.synchronize()
    err = max_err(host(ot), oracle_out(drafts_h[-1][0]))          # the last draft step itself
    assert err <= F32_TOL, err
    assert rt[0].ring_len == 15
    K.rswa_rollback_to(test, rt, 0, cp)
    model.rollback_to(mcp)
    assert (rt[0].ring_len, rt[0].ring_pos, rt[0].writes, test.len[0]) == (9, 9, 9, pf + 9)
    assert (model.ring_len, model.ring_pos, model.writes) == (9, 9, 9)
    torch.cuda.synchronize()
    stale = host(drafts[0][1])[0]
    if kind == K.KIND_F32:
        assert np.array_equal(host(test.view("k"))[0][:, pf + 9], stale)      # stale, never read
    else:
        codes = np.stack([oracle.quant_row_i8(stale[g])[0] for g in range(nh)])
        assert np.array_equal(host(test.view("kq"))[0][:, pf + 9], codes)
    for t in range(9, 14):
        q, k, v = acc[t]
        K.rswa_decode(test, rt, nh, q, k, v, ot)
        K.rswa_decode(ctrl, rc, nh, q, k, v, oc)
        rows[("a", t)] = (acc_h[t][1][0], acc_h[t][2][0])
        model.write(("a", t))
        torch.cuda.synchronize()
        assert np.array_equal(host(ot).view(np.uint32), host(oc).view(np.uint32)), t
        err = max_err(host(ot), oracle_out(acc_h[t][0]))
        say("  rollback kind %d step %d max err %.3g" % (kind, t, err))
        assert err <= F32_TOL, (t, err)
    n = pf + 14
    for nm in BUFS[kind]:
        a, b = host(test.view(nm))[:, :, :n], host(ctrl.view(nm))[:, :, :n]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), nm
    # the abandoned branch's checkpoint no longer matches
    with pytest.raises(K.KvqError):
        K.rswa_rollback_to(test, rt, 0, cp)
