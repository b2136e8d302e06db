"""The f32 decode of groups of 1 over long and short segments, against the
oracle's f64 attention, on workspaces filled with 0xFF bytes (NaN as f32)
and with random bytes beforehand: the split's partials ([P3] fold) must
never read a workspace byte that the call did not write first, and the
number of partials per (sequence, head) -- printed for each case -- ranges
from 1 to more than a hundred."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import F32_TOL, THREADS, append_rows, dev, host, max_err, say
from int8_kv_cache_decode_amd import kvq as K

pytestmark = pytest.mark.gpu


def simds() -> int:
    return 4 * torch.cuda.get_device_properties(0).multi_processor_count


def max_parts(lens, n_heads) -> int:
    """Most partials of one (sequence, head) segment under the launcher's
    split (for the printed case description): one share per SIMD (one tile
    per share when a launch has fewer than two tiles per SIMD), shares cut
    evenly from the tile stream."""
    nt = [(n + 15) // 16 for n in lens]
    T = sum(nt) * n_heads
    W = simds()
    W = T if T < 2 * W else W
    W = min(W, T)
    owner = lambda t: ((t + 1) * W - 1) // T
    best, base = 1, 0
    for n in nt:
        for _ in range(n_heads):
            if n:
                best = max(best, owner(base + n - 1) - owner(base) + 1)
            base += n
    return best


def f32_case(lens, n_heads, seed):
    r = np.random.default_rng(seed)
    c = K.KvCache(K.KIND_F32, len(lens), n_heads, max(lens))
    units = []
    for b, n in enumerate(lens):
        k = r.standard_normal((n, n_heads, 128)).astype(np.float32)
        v = r.standard_normal((n, n_heads, 128)).astype(np.float32)
        append_rows(c, b, k, v)
        units.append([("f32", np.ascontiguousarray(k[:, g]), np.ascontiguousarray(v[:, g])) for g in range(n_heads)])
    return c, units


def garbage_ws(c, n_q_heads, fill):
    ws = torch.empty(K.kvq_workspace_bytes(c, n_q_heads), dtype=torch.uint8, device="cuda")
    if fill == "ff":
        ws.fill_(0xFF)
    else:
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=torch.Generator().manual_seed(fill)))
    return ws


def run_and_check(c, units, n_heads, q, ws, **kw):
    out = torch.full(q.shape, float("nan"), device="cuda")
    if kw:
        opts = K.DecodeOpts(first=kw.get("first"), sinks=None if kw.get("sinks") is None else dev(kw["sinks"]))
        K.decode_attn_f32_ex(c, n_heads, dev(q), out, opts, ws=ws)
    else:
        K.decode_attn_f32(c, n_heads, dev(q), out, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.decode(q, units, n_heads, threads=THREADS, **kw)
    err = max_err(host(out), ref)
    assert err <= F32_TOL, err
    return err


def test_f32_long_segments_on_garbage_workspaces():
    """Ten heads of 32773 rows (about 103 partials per head), three calls on
    a workspace of 0xFF bytes and three on random bytes, each with a new
    query."""
    lens, H = [32773], 10
    say("case: f32 long, max parts", max_parts(lens, H))
    c, units = f32_case(lens, H, 1400)
    r = np.random.default_rng(1401)
    for fill in ("ff", 7):
        ws = garbage_ws(c, H, fill)
        for call in range(3):
            q = (r.standard_normal((1, H, 128)) * (1 + 2 * call)).astype(np.float32)
            say("  fill", fill, "call", call, "err", run_and_check(c, units, H, q, ws))


@pytest.mark.parametrize("n_heads", [9, 10, 12])
def test_f32_partials_per_head(n_heads):
    """20000 rows per head over 9, 10 or 12 heads: about 115, 104 and 86
    partials per head."""
    lens = [20000]
    say("case: f32 heads", n_heads, "max parts", max_parts(lens, n_heads))
    c, units = f32_case(lens, n_heads, 1410 + n_heads)
    q = np.random.default_rng(1420 + n_heads).standard_normal((1, n_heads, 128)).astype(np.float32)
    run_and_check(c, units, n_heads, q, garbage_ws(c, n_heads, "ff"))


def test_f32_sinks_and_window_on_garbage_workspace():
    """Two sequences x 10 heads with sink logits and a visible-row start."""
    lens, H = [30000, 12345], 10
    say("case: f32 sinks/window, max parts", max_parts(lens, H))
    c, units = f32_case(lens, H, 1430)
    r = np.random.default_rng(1431)
    q = r.standard_normal((2, H, 128)).astype(np.float32)
    sinks = r.standard_normal(H).astype(np.float32) * 3
    ws = garbage_ws(c, H, 11)
    run_and_check(c, units, H, q, ws, sinks=sinks)
    run_and_check(c, units, H, q, ws, first=np.array([5000, 12000], np.int32), sinks=sinks)
    run_and_check(c, units, H, q, ws, first=np.array([29999, 0], np.int32))


def test_f32_many_short_sequences_two_launches():
    """130 sequences (two launches sharing one workspace) of 1..600 rows x 2
    heads: most segments lie inside one share (one partial), the others span
    a few."""
    r = np.random.default_rng(1440)
    lens = [int(x) for x in r.integers(1, 601, 130)]
    H = 2
    say("case: f32 short x130, max parts", max_parts(lens[:128], H))
    c, units = f32_case(lens, H, 1441)
    ws = garbage_ws(c, H, "ff")
    for call in range(2):
        q = r.standard_normal((130, H, 128)).astype(np.float32)
        run_and_check(c, units, H, q, ws)
