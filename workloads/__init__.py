"""Seeded synthetic inputs for the decode-attention workloads.

This module holds no arithmetic of the method (no attention, no codec): only
a counter-based random generator and the recipes that shape its output into
the workloads' tensors.  Both the HIP path's tests/benchmark and the CPU
oracle's tests take their inputs from here; nothing else is shared.

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit finaliser constants of Vigna's
public-domain splitmix64.c).  Output i of stream `key` is
mix(key + (i + 1) * 0x9E3779B97F4A7C15).  Uniforms take the top 53 bits;
normals use Box-Muller in float64 and are rounded to float32 once.

Workloads (sizes of the pages' decode paths):
  rswa_f32        R-SWA MHA: 10 heads x 128, reference block of 256 rows,
                  165 ring writes (ring_pos 37 after wrap-around)
  gqa_f32         32 Q / 8 KV heads x 128, context 4096, KV groups 2 and 5 dead
  gqa_q8          32 Q / 8 KV heads x 128, context 8192, per-channel factors
                  log-uniform in [0.25, 8], all rows through the q8 quantiser
  rswa_long_f32   R-SWA MHA: 10 heads x 128, reference block 32640 rows,
                  500 ring writes (ring full, ring_pos 116)
  batched_q8      64 sequences, 32 Q / 8 KV heads x 128, context lengths
                  uniform in [1024, 32768], factors as gqa_q8
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1

# stream tags
TAG_Q, TAG_K, TAG_V, TAG_FK, TAG_FV, TAG_LEN, TAG_RK, TAG_RV, TAG_RQ = range(1, 10)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def key(seed: int, *tags: int) -> int:
    """Derive an independent stream key from a seed and integer tags."""
    k = seed & _MASK
    for t in tags:
        k = _mix_int(k ^ _mix_int((t + 0x9E3779B97F4A7C15) & _MASK))
    return k


def u64(k: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start..start+n-1 of the SplitMix64 stream with state `k`."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        return _mix(np.uint64(k) + i * _GAMMA)


def uniform(k: int, n: int) -> np.ndarray:
    """float64 uniforms in [0, 1)."""
    return (u64(k, n) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(k: int, shape) -> np.ndarray:
    """float64 N(0, 1) by Box-Muller (both branches used)."""
    n = int(np.prod(shape))
    return _normal_from(k, 0, n).reshape(shape)


def normal_f32(k: int, shape) -> np.ndarray:
    return normal(k, shape).astype(np.float32)


def log_uniform(k: int, shape, lo: float, hi: float) -> np.ndarray:
    u = uniform(k, int(np.prod(shape))).reshape(shape)
    return np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def int_uniform(k: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive."""
    u = uniform(k, n)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


# --------------------------------------------------------------------------
# Workload recipes
# --------------------------------------------------------------------------
@dataclass
class GqaSpec:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kind: str                       # "f32" or "q8"
    ctx: Optional[int] = None       # fixed context length, or None
    len_range: Optional[Tuple[int, int]] = None
    dead: Tuple[int, ...] = ()
    factor_range: Optional[Tuple[float, float]] = None

    def lengths(self) -> np.ndarray:
        if self.ctx is not None:
            return np.full(self.batch, self.ctx, np.int64)
        lo, hi = self.len_range
        return int_uniform(key(self.seed, TAG_LEN), self.batch, lo, hi)

    def alive(self) -> np.ndarray:
        a = np.ones(self.n_kv_heads, np.uint8)
        for g in self.dead:
            a[g] = 0
        return a

    def capacity(self) -> int:
        return int(self.lengths().max())

    def query(self) -> np.ndarray:
        """q [B][Hq][hd] ~ N(0, 1)."""
        return normal_f32(key(self.seed, TAG_Q), (self.batch, self.n_q_heads, self.head_dim))

    def kv_rows(self, b: int, start: int = 0, count: Optional[int] = None):
        """K, V rows of sequence b as the append call takes them:
        [count][Hkv][hd] f32 each, rows start..start+count-1.  Dead groups
        carry values too (the append skips them)."""
        n = int(self.lengths()[b])
        if count is None:
            count = n - start
        shape = (count, self.n_kv_heads, self.head_dim)
        per_row = self.n_kv_heads * self.head_dim
        kk = key(self.seed, TAG_K, b)
        kv = key(self.seed, TAG_V, b)
        k = _normal_range(kk, start * per_row, count * per_row).reshape(shape)
        v = _normal_range(kv, start * per_row, count * per_row).reshape(shape)
        if self.factor_range is not None:
            fk, fv = self.factors(b)
            k = k * fk[None, :, :]
            v = v * fv[None, :, :]
        return k.astype(np.float32), v.astype(np.float32)

    def factors(self, b: int):
        """Per-channel factors [Hkv][hd] for K and for V of sequence b,
        log-uniform in factor_range, constant over positions."""
        lo, hi = self.factor_range
        shape = (self.n_kv_heads, self.head_dim)
        return (log_uniform(key(self.seed, TAG_FK, b), shape, lo, hi),
                log_uniform(key(self.seed, TAG_FV, b), shape, lo, hi))


def _normal_range(k: int, start: int, n: int) -> np.ndarray:
    """Elements start..start+n-1 of the normal stream `k` (equal to the same
    slice of normal(k, ...) drawn from position 0)."""
    s0 = start - (start % 2)
    return _normal_from(k, s0, (start - s0) + n)[start - s0:]


def _normal_from(k: int, s0: int, n: int) -> np.ndarray:
    """n normals starting at stream element s0 (s0 even: Box-Muller element j
    uses uniforms 2*(j//2) and 2*(j//2)+1)."""
    m = (n + 1) // 2
    u = (u64(k, 2 * m, start=s0) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    u1 = 1.0 - u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * math.pi * u2
    z = np.empty(2 * m, np.float64)
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    return z[:n]


@dataclass
class RswaSpec:
    name: str
    seed: int
    n_heads: int
    head_dim: int
    prefill: int
    writes: int
    window: int = 128

    def reference(self):
        """Reference block K, V: [n_heads][prefill][hd] f32 (head-major)."""
        shape = (self.n_heads, self.prefill, self.head_dim)
        return (normal_f32(key(self.seed, TAG_K), shape),
                normal_f32(key(self.seed, TAG_V), shape))

    def step(self, t: int):
        """Decode step t (t = 0, 1, ...): q, k, v each [n_heads][hd] f32."""
        shape = (self.n_heads, self.head_dim)
        return (normal_f32(key(self.seed, TAG_RQ, t), shape),
                normal_f32(key(self.seed, TAG_RK, t), shape),
                normal_f32(key(self.seed, TAG_RV, t), shape))


WORKLOADS: Dict[str, object] = {
    "rswa_f32": RswaSpec("rswa_f32", 0x5EED0001, 10, 128, 256, 165),
    "gqa_f32": GqaSpec("gqa_f32", 0x5EED0002, 1, 32, 8, 128, "f32", ctx=4096, dead=(2, 5)),
    "gqa_q8": GqaSpec("gqa_q8", 0x5EED0003, 1, 32, 8, 128, "q8", ctx=8192,
                      factor_range=(0.25, 8.0)),
    "rswa_long_f32": RswaSpec("rswa_long_f32", 0x5EED0004, 10, 128, 32640, 500),
    "batched_q8": GqaSpec("batched_q8", 0x5EED0005, 64, 32, 8, 128, "q8",
                          len_range=(1024, 32768), factor_range=(0.25, 8.0)),
}


def get(name: str):
    return WORKLOADS[name]
