"""Helpers for the GPU parity tests: build caches through the C ABI from the
seeded workloads, read device storage back, and build the oracle's side from
the same inputs.  The HIP path and the oracle share nothing but the inputs."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from int8_kv_cache_decode_amd import kvq as K

F32_TOL = 1e-5          # max-abs bound on f32 outputs against the f64 oracle
THREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def append_rows(cache: K.KvCache, seq: int, k: np.ndarray, v: np.ndarray, chunks=None):
    """Append rows [n][Hkv][128] through the ABI, optionally in chunks."""
    n = k.shape[0]
    fn = {K.KIND_F32: K.kv_append_f32, K.KIND_Q8: K.kv_append_q8, K.KIND_I8: K.kv_append_i8}[cache.kind]
    bounds = [0] + list(chunks or []) + [n]
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if hi > lo:
            fn(cache, seq, hi - lo, dev(k[lo:hi]), dev(v[lo:hi]))


def oracle_q8_heads(k: np.ndarray, v: np.ndarray, alive, cap=None):
    """Per live KV head g: an oracle Q8Head holding rows k[:, g], v[:, g]."""
    n, hkv, _ = k.shape
    heads = [None] * hkv

    def one(g):
        if alive[g]:
            h = oracle.Q8Head(cap=cap or max(n, 1))
            if n:
                h.append(k[:, g], v[:, g])
            heads[g] = h

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, range(hkv)))
    return heads


def assert_codes_equal(cache: K.KvCache, b: int, heads, alive, n: int):
    """Bit-exact q8 storage of sequence b against oracle heads."""
    kq, ks = host(cache.view("kq")[b]), host(cache.view("ks")[b])
    vq, vs = host(cache.view("vq")[b]), host(cache.view("vs")[b])
    kcol, vcol = host(cache.view("kcol")[b]), host(cache.view("vcol")[b])
    slot = 0
    for g, h in enumerate(heads):
        if not alive[g]:
            continue
        assert h.n == n
        assert np.array_equal(kq[slot, :n], h.kq[:n]), ("kq", b, g, first_diff(kq[slot, :n], h.kq[:n]))
        assert np.array_equal(ks[slot, :n].view(np.uint32), h.ks[:n].view(np.uint32)), ("ks", b, g)
        assert np.array_equal(vq[slot, :n], h.vq[:n]), ("vq", b, g, first_diff(vq[slot, :n], h.vq[:n]))
        assert np.array_equal(vs[slot, :n].view(np.uint32), h.vs[:n].view(np.uint32)), ("vs", b, g)
        if h.frozen:
            assert bool(cache.frozen[b])
            assert np.array_equal(kcol[slot].view(np.uint32), h.kcol.view(np.uint32)), ("kcol", b, g)
            assert np.array_equal(vcol[slot].view(np.uint32), h.vcol.view(np.uint32)), ("vcol", b, g)
        else:
            assert not cache.frozen[b]
        slot += 1


def first_diff(a, b):
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return None
    i = tuple(idx[0])
    return i, a[i], b[i], len(idx)


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got.astype(np.float64) - ref))) if got.size else 0.0
