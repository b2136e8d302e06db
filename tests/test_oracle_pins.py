"""Pins the CPU oracle to things other than itself (CPU only).

Every check here compares the oracle against something the pages or the
mathematics fix independently of the oracle's code: values the pages print
for worked examples (tests/golden/, each cited), closed forms, invariants,
a library routine that computes the same definition (torch's
scaled_dot_product_attention in float64), and exact rational arithmetic for
the f32 codec.

Pages:
  [P1] cortiq-engine 0.3.4, src/cortiq_engine/kv_cache.rs
  [P2] cortiq-engine 0.8.49, src/cortiq_engine/kv_cache.rs
  [P3] franken_ocr 0.8.0, src/native_engine/rswa.rs
"""
import decimal
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

HD = 128


def bits_f32(h: str) -> float:
    return struct.unpack("<f", struct.pack("<I", int(h, 16)))[0]


def f32_round(x: Fraction) -> float:
    """Round an exact rational to the nearest float32, ties to even."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                         # subnormal range keeps the exponent
    m = a / (Fraction(2) ** (e - 23))        # in [2^23, 2^24) for normals
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * Fraction(2) ** (e - 23)
    return sign * float(np.float32(float(val)))


def half_away(x: float) -> int:
    return int(math.copysign(math.floor(abs(x) + 0.5), x))


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Attention (float64, by definition)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,hd,hpk", [(1, 4, 1), (2, 4, 1), (3, 32, 2), (9, 128, 1),
                                      (9, 128, 4), (300, 128, 4), (57, 32, 3)])
def test_attention_matches_library_sdpa(n, hd, hpk):
    """Library routine computing the same definition: torch SDPA in float64
    with its default scale 1/sqrt(hd)."""
    r = rng(1000 + n * 7 + hd + hpk)
    q = r.standard_normal((hpk, hd)).astype(np.float32)
    k = r.standard_normal((n, hd)).astype(np.float32) * 2
    v = r.standard_normal((n, hd)).astype(np.float32)
    got = oracle.attend_f32(q, k, v)
    tq = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
    tk = torch.from_numpy(k.astype(np.float64))[None, None].expand(1, hpk, n, hd).contiguous()
    tv = torch.from_numpy(v.astype(np.float64))[None, None].expand(1, hpk, n, hd).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_empty_rows_give_zero():
    """[P1] attend_group: stored == 0 -> output filled with 0."""
    q = np.ones((4, HD), np.float32)
    out = oracle.attend_f32(q, np.zeros((0, HD), np.float32), np.zeros((0, HD), np.float32))
    assert out.shape == (4, HD) and not out.any()


def _e(dim, value, hd=HD):
    x = np.zeros(hd, np.float32)
    x[dim] = value
    return x


def test_worked_values_from_rswa_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rswa_worked_values.json")))
    sk = g["single_key"]
    out = oracle.attend_f32(_e(sk["q"]["dim"], sk["q"]["value"]),
                            _e(sk["k0"]["dim"], sk["k0"]["value"])[None],
                            np.full((1, HD), sk["v"], np.float32))
    assert np.all(out == sk["expected"])          # a single key has weight exactly 1

    eq = g["equal_scores"]
    k = np.stack([_e(eq["k"]["dim"], eq["k"]["value"])] * 2)
    v = np.stack([np.full(HD, x, np.float32) for x in eq["v_rows"]])
    out = oracle.attend_f32(_e(eq["q"]["dim"], eq["q"]["value"]), k, v)
    np.testing.assert_allclose(out, eq["expected"], rtol=0, atol=1e-15)

    rp = g["reference_plus_ring"]
    k = np.stack([_e(rp["ref_key_dim"], 1.0), _e(rp["ring_key_dim"], 1.0)])
    v = np.stack([np.full(HD, rp["ref_v"], np.float32), np.full(HD, rp["ring_v"], np.float32)])
    q = _e(0, rp["q_e0"])
    out = oracle.attend_f32(q, k, v)
    # the page's printed digits
    assert abs(out[0] - rp["printed_output"]) < rp["printed_digits_tolerance"]
    w = oracle.weights_f32(q, k)
    assert abs(w[1] - rp["printed_ring_weight"]) < rp["printed_digits_tolerance"]
    assert abs(w[0] - rp["printed_ref_weight"]) < rp["printed_digits_tolerance"]
    # the page's closed form, two keys: logistic of the score gap
    e = math.exp(rp["q_e0"] / math.sqrt(HD))
    np.testing.assert_allclose(out, (e * rp["ring_v"] + rp["ref_v"]) / (e + 1), rtol=0, atol=1e-14)


def test_weights_sum_to_one_and_constant_values():
    r = rng(7)
    for n in (1, 5, 64, 1000):
        q = r.standard_normal(HD).astype(np.float32) * 3
        k = r.standard_normal((n, HD)).astype(np.float32)
        w = oracle.weights_f32(q, k)
        assert abs(w.sum() - 1.0) < 1e-12 and np.all(w > 0)
        out = oracle.attend_f32(q, k, np.ones((n, HD), np.float32))
        np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_permutation_invariance_and_convex_hull():
    r = rng(8)
    n = 77
    q = r.standard_normal((4, HD)).astype(np.float32)
    k = r.standard_normal((n, HD)).astype(np.float32)
    v = r.standard_normal((n, HD)).astype(np.float32)
    perm = r.permutation(n)
    a = oracle.attend_f32(q, k, v)
    b = oracle.attend_f32(q, k[perm], v[perm])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    assert np.all(a <= v.max(axis=0) + 1e-12) and np.all(a >= v.min(axis=0) - 1e-12)


def test_zero_query_gives_mean_and_sharp_query_gives_argmax():
    r = rng(9)
    n = 33
    k = r.standard_normal((n, HD)).astype(np.float32)
    v = r.standard_normal((n, HD)).astype(np.float32)
    out = oracle.attend_f32(np.zeros(HD, np.float32), k, v)
    np.testing.assert_allclose(out, v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-13)
    # a query far along key j: softmax collapses onto row j
    j = 17
    q = (k[j] * 200.0).astype(np.float32)
    out = oracle.attend_f32(q, k, v)
    np.testing.assert_allclose(out, v[j], rtol=0, atol=1e-9)


def test_linearity_in_values():
    r = rng(10)
    n = 40
    q = r.standard_normal(HD).astype(np.float32)
    k = r.standard_normal((n, HD)).astype(np.float32)
    v1 = r.standard_normal((n, HD)).astype(np.float32)
    v2 = r.standard_normal((n, HD)).astype(np.float32)
    a = oracle.attend_f32(q, k, v1) * 0.5 + oracle.attend_f32(q, k, v2) * 2.0
    b = oracle.attend_f32(q, k, (v1.astype(np.float64) * 0.5 + v2 * 2.0).astype(np.float32))
    # (the combined V is rounded to f32 once, so allow that rounding)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-6)


def test_gqa_mapping_and_dead_groups():
    """[P1] attend_group: Q head h reads KV group h // hpk; dead groups
    store nothing and their Q heads output zeros.  Checked against torch SDPA
    with K/V repeated per Q head (float64)."""
    r = rng(11)
    B, Hq, Hkv, n = 2, 8, 4, 23
    hpk = Hq // Hkv
    q = r.standard_normal((B, Hq, HD)).astype(np.float32)
    k = r.standard_normal((B, Hkv, n, HD)).astype(np.float32)
    v = r.standard_normal((B, Hkv, n, HD)).astype(np.float32)
    dead = {1}
    units = [[None if g in dead else ("f32", k[b, g], v[b, g]) for g in range(Hkv)] for b in range(B)]
    out = oracle.decode(q, units, Hkv, threads=3)
    tq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(hpk, dim=1)
    tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(hpk, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, :, 0, :].numpy()
    for h in range(Hq):
        if h // hpk in dead:
            assert not out[:, h].any()
        else:
            np.testing.assert_allclose(out[:, h], ref[:, h], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# q8_2f codec (IEEE f32, step by step)
# ---------------------------------------------------------------------------
def test_quant_row_half_away_fixture(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "q8_2f_quant_fixtures.json")))["half_away_row"]
    x = np.zeros(fx["head_dim"], np.float32)
    x[: len(fx["row_prefix"])] = fx["row_prefix"]
    m = len(fx["k_codes_prefix"])
    q, s = oracle.quant_row(x, None, 32)
    assert s[0] == fx["k_group0_scale"]
    assert list(q[:m]) == fx["k_codes_prefix"] and not q[m:].any()
    tiny = np.float32(fx["zero_group_scale_f32_of"])
    assert np.all(s[1:] == tiny)
    qv, sv = oracle.quant_row(x, None, fx["head_dim"])
    assert sv.shape == (1,) and sv[0] == fx["v_scale"]
    assert list(qv[:m]) == fx["v_codes_prefix"] and not qv[m:].any()


def test_quant_row_divides_and_rounds_half_away(golden_dir):
    """Expected codes from exact rational arithmetic: s = f32(absmax/127),
    code = half_away(f32(x/s)).  Each case also shows which wrong reading it
    rules out (multiplying by f32(1/s), or rounding ties to even)."""
    fx = json.load(open(os.path.join(golden_dir, "q8_2f_quant_fixtures.json")))["division_cases"]
    ruled_out = set()
    for case in fx["cases"]:
        a, x = bits_f32(case["absmax_bits"]), bits_f32(case["x_bits"])
        s = f32_round(Fraction(a) / 127)
        quot = f32_round(Fraction(x) / Fraction(s))
        want = max(-127, min(127, half_away(quot)))
        recip = f32_round(Fraction(x) * Fraction(f32_round(1 / Fraction(s))))
        if half_away(recip) != want:
            ruled_out.add("reciprocal")
        if quot == math.floor(quot) + 0.5 and round(quot) != want:   # Python round = ties-even
            ruled_out.add("ties-even")
        row = np.zeros(HD, np.float32)
        row[0], row[1] = a, x
        q, sc = oracle.quant_row(row, None, 32)
        assert sc[0] == np.float32(s)
        assert q[1] == want, (case, q[1], want)
        assert q[0] == 127
    assert ruled_out == {"reciprocal", "ties-even"}


def test_quant_row_against_exact_rationals_random():
    """Random rows (with and without a column field): every scale and code
    equals the exact-rational computation of the page's steps."""
    r = rng(12)
    for trial in range(6):
        x = (r.standard_normal(HD) * r.uniform(0.01, 50)).astype(np.float32)
        col = None if trial % 2 == 0 else r.uniform(0.2, 9, HD).astype(np.float32)
        for group in (32, HD):
            q, s = oracle.quant_row(x, col, group)
            resid = [Fraction(float(x[d])) if col is None
                     else Fraction(f32_round(Fraction(float(x[d])) / Fraction(float(col[d]))))
                     for d in range(HD)]
            for gi, g0 in enumerate(range(0, HD, group)):
                am = max(abs(v) for v in resid[g0:g0 + group])
                sc = max(f32_round(am / 127), float(np.float32(1e-12)))
                assert s[gi] == np.float32(sc)
                for d in range(g0, g0 + group):
                    want = max(-127, min(127, half_away(f32_round(resid[d] / Fraction(sc)))))
                    assert q[d] == want


def test_quant_row_invariants():
    r = rng(13)
    for _ in range(20):
        x = (r.standard_normal(HD) * r.uniform(1e-3, 1e3)).astype(np.float32)
        q, s = oracle.quant_row(x, None, 32)
        for gi in range(4):
            g = slice(32 * gi, 32 * gi + 32)
            # the group's absmax element maps to +-127
            j = 32 * gi + int(np.argmax(np.abs(x[g])))
            assert abs(int(q[j])) == 127 and np.sign(q[j]) == np.sign(x[j])
            # round-trip bound |x - q*s| <= s/2 (plus the division's rounding)
            err = np.abs(x[g].astype(np.float64) - q[g].astype(np.float64) * float(s[gi]))
            assert np.all(err <= 0.5 * float(s[gi]) * (1 + 2 ** -20))
        # power-of-two scaling is exact: codes unchanged, scales scaled
        for e in (-3, 5):
            q2, s2 = oracle.quant_row((x * np.float32(2.0 ** e)).astype(np.float32), None, 32)
            assert np.array_equal(q, q2) and np.array_equal(s * np.float32(2.0 ** e), s2)


def test_quant_row_lossless_integers_exhaustive():
    """Rows of integers whose groups contain +-127 have scale 1 and codes equal
    to the values: every code -127..127 round-trips."""
    codes = np.arange(-127, 128)
    full = np.concatenate([codes, codes[::-1], codes])[: 3 * HD]
    for start in range(0, len(full) - HD + 1, HD):
        x = full[start:start + HD].astype(np.float32).copy()
        for gi in range(4):
            x[32 * gi] = 127.0
        q, s = oracle.quant_row(x, None, 32)
        assert np.all(s == 1.0) and np.array_equal(q.astype(np.float32), x)
    covered = set()
    for start in range(0, len(full) - HD + 1, HD):
        covered |= set(full[start:start + HD].tolist())
    assert covered == set(range(-127, 128))


def test_zero_group_scale():
    q, s = oracle.quant_row(np.zeros(HD, np.float32), None, 32)
    assert not q.any() and np.all(s == np.float32(1e-12))
    q, s = oracle.quant_row(np.zeros(HD, np.float32), np.full(HD, 3.0, np.float32), HD)
    assert not q.any() and s[0] == np.float32(1e-12)


def _lossless_rows(r, n, c=None):
    """n rows of integers; every K group and every row contains +-127."""
    if c is None:
        x = r.integers(-127, 128, size=(n, HD)).astype(np.float32)
    else:
        x = (np.where(r.random((n, HD)) < 0.5, -1.0, 1.0) * c[None, :]).astype(np.float32)
    x[:, ::32] = np.where(r.random((n, 4)) < 0.5, -127.0, 127.0)
    return x


def test_freeze_constant_magnitude_closed_form():
    """Channels of constant magnitude c_d over 64 lossless rows: the field is
    exactly c_d, every requantised residual is +-1, so every code is +-127 and
    every scale is f32(1/127) ([P1] freeze_cols on closed-form rows)."""
    r = rng(14)
    c = r.integers(1, 128, size=HD).astype(np.float64)
    c[::32] = 127.0
    k = _lossless_rows(r, 65, c)
    v = _lossless_rows(r, 65, c)
    h = oracle.Q8Head(cap=80, hd=HD)
    h.append(k[:64], v[:64])
    assert h.n == 64 and not h.frozen                      # 64 rows: not yet frozen
    assert np.array_equal(h.kq[:64].astype(np.float32), k[:64]) and np.all(h.ks[:64] == 1.0)
    h.append(k[64:65], v[64:65])                            # the 65th append freezes first
    assert h.frozen and h.n == 65
    assert np.array_equal(h.kcol, c.astype(np.float32)) and np.array_equal(h.vcol, c.astype(np.float32))
    inv127 = np.float32(f32_round(Fraction(1, 127)))
    code = half_away(f32_round(Fraction(1) / Fraction(float(inv127))))
    assert code == 127
    for p in range(65):                                     # row 64 against the frozen field too
        assert np.array_equal(h.kq[p], (np.sign(k[p]) * 127).astype(np.int8))
        assert np.array_equal(h.vq[p], (np.sign(v[p]) * 127).astype(np.int8))
        assert np.all(h.ks[p] == inv127) and h.vs[p] == inv127


def _sqrt_f32_exact(x: Fraction) -> float:
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        d = (decimal.Decimal(x.numerator) / decimal.Decimal(x.denominator)).sqrt()
    return f32_round(Fraction(d))


def test_freeze_rms_exact_sums():
    """Lossless integer rows: sum of squares is exact in f32, so the field is
    the correctly rounded sqrt(sum/64), floored at 1e-6."""
    r = rng(15)
    k = _lossless_rows(r, 65)
    v = _lossless_rows(r, 65)
    k[:64, 5] = 0.0                                         # an all-zero channel -> 1e-6
    h = oracle.Q8Head(cap=70, hd=HD)
    h.append(k, v)
    for name, x, col in (("k", k, h.kcol), ("v", v, h.vcol)):
        for d in range(HD):
            s = int(np.sum(x[:64, d].astype(np.int64) ** 2))
            want = max(_sqrt_f32_exact(Fraction(s, 64)), float(np.float32(1e-6)))
            assert col[d] == np.float32(want), (name, d)


def test_freeze_rms_rounds_each_operation():
    """Non-integer rows: the field follows the page's f32 steps exactly --
    x^ = f32(code*scale), acc = f32(acc + f32(x^*x^)) sequentially over rows
    (a multiply and an add, each rounded; no fused multiply-add),
    col = max(f32(sqrt(f32(acc/n))), 1e-6).  Recomputed with exact rationals;
    the fused variant is also computed to show the case separates the two."""
    r = rng(20)
    k = (r.standard_normal((65, HD)) * r.uniform(0.3, 7, HD)).astype(np.float32)
    v = (r.standard_normal((65, HD)) * 2.5).astype(np.float32)
    h = oracle.Q8Head(cap=65, hd=HD)
    h.append(k[:64], v[:64])
    kq0, ks0 = h.kq[:64].copy(), h.ks[:64].copy()
    h.append(k[64:], v[64:])
    fused_differs = False
    for d in range(0, HD, 3):
        acc = Fraction(0)
        acc_fma = Fraction(0)
        for p in range(64):
            xh = Fraction(f32_round(Fraction(int(kq0[p, d])) * Fraction(float(ks0[p, d // 32]))))
            acc = Fraction(f32_round(acc + Fraction(f32_round(xh * xh))))
            acc_fma = Fraction(f32_round(acc_fma + xh * xh))
        want = max(_sqrt_f32_exact(Fraction(f32_round(acc / 64))), float(np.float32(1e-6)))
        assert h.kcol[d] == np.float32(want), d
        fused_differs |= acc != acc_fma
    assert fused_differs


def test_freeze_requantises_dequantised_rows():
    """After the freeze, rows 0..63 are the quantisation of the DEQUANTISED
    rows against the field; later rows quantise the raw input against it."""
    r = rng(16)
    k = (r.standard_normal((70, HD)) * 3).astype(np.float32)
    v = (r.standard_normal((70, HD)) * 3).astype(np.float32)
    h = oracle.Q8Head(cap=70, hd=HD)
    h.append(k[:64], v[:64])
    kq0, ks0 = h.kq[:64].copy(), h.ks[:64].copy()
    h.append(k[64:], v[64:])
    xh = (kq0.astype(np.float32) * np.repeat(ks0, 32, axis=1)).astype(np.float32)
    for p in (0, 31, 63):
        q, s = oracle.quant_row(xh[p], h.kcol, 32)
        assert np.array_equal(q, h.kq[p]) and np.array_equal(s, h.ks[p])
    for p in (64, 69):
        q, s = oracle.quant_row(k[p], h.kcol, 32)
        assert np.array_equal(q, h.kq[p]) and np.array_equal(s, h.ks[p])
        q, s = oracle.quant_row(v[p], h.vcol, HD)
        assert np.array_equal(q, h.vq[p]) and s[0] == h.vs[p]


def test_chunked_append_equals_row_by_row_and_explicit_freeze():
    r = rng(17)
    k = (r.standard_normal((130, HD)) * 2).astype(np.float32)
    v = (r.standard_normal((130, HD)) * 2).astype(np.float32)
    a = oracle.Q8Head(cap=130)
    for p in range(130):
        a.append(k[p:p + 1], v[p:p + 1])
    b = oracle.Q8Head(cap=130)
    for lo, hi in ((0, 7), (7, 64), (64, 65), (65, 130)):
        b.append(k[lo:hi], v[lo:hi])
    c = oracle.Q8Head(cap=130)
    c.append(k, v)
    for o in (b, c):
        for f in ("kq", "ks", "vq", "vs", "kcol", "vcol"):
            assert np.array_equal(getattr(a, f), getattr(o, f)), f
    # an explicit freeze is a no-op once frozen, and freezes early otherwise
    assert not a.freeze()
    e = oracle.Q8Head(cap=40)
    e.append(k[:40], v[:40])
    assert not e.frozen and e.freeze() and e.frozen and not e.freeze()


def test_q8_attention_within_page_grid_bound():
    """[P1] test q8_attend_matches_f32_within_grid: 100 positions (crossing the
    freeze), 2 heads x 32 channels of the page's modular pattern with even
    channels x4 and odd x0.25; q8 output within 0.03*max|o| + 1e-3 of f32 and
    probabilities within 0.02."""
    heads, hd = 2, 32

    def synth(p, salt):
        i = np.arange(heads * hd)
        x = ((i * 31 + p * 17 + salt * 7 + 3) % 97).astype(np.float32) / np.float32(97.0) - np.float32(0.5)
        return np.where(i % 2 == 0, x * np.float32(4.0), x * np.float32(0.25)).astype(np.float32)

    K = np.stack([synth(p, 1) for p in range(100)]).reshape(100, heads, hd)
    V = np.stack([synth(p, 2) for p in range(100)]).reshape(100, heads, hd)
    q = (((np.arange(hd) * 13 + 5) % 89).astype(np.float32) / np.float32(89.0) - np.float32(0.5)).astype(np.float32)
    for g in range(heads):
        h = oracle.Q8Head(cap=100, hd=hd)
        h.append(K[:, g], V[:, g])
        assert h.frozen
        of = oracle.attend_f32(q, K[:, g], V[:, g])
        o8 = oracle.attend_q8(q, h)
        scale = max(np.abs(of).max(), 1e-6)
        assert np.all(np.abs(of - o8) <= scale * 0.03 + 1e-3)
        pf = oracle.weights_f32(q, K[:, g])
        p8 = oracle.weights_f32(q, h.dequant_k().astype(np.float32))
        assert np.all(np.abs(pf - p8) < 0.02)


def test_q8_attention_equals_attention_on_dequantised_rows():
    """attend_q8 is attention over K^ = code*scale*col, V^ = code*scale*col."""
    r = rng(18)
    h = oracle.Q8Head(cap=100)
    h.append((r.standard_normal((100, HD)) * 4).astype(np.float32),
             (r.standard_normal((100, HD)) * 4).astype(np.float32))
    q = r.standard_normal((4, HD)).astype(np.float32)
    got = oracle.attend_q8(q, h)
    kk, vv = h.dequant_k(), h.dequant_v()
    tq = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
    tk = torch.from_numpy(kk)[None, None].expand(1, 4, 100, HD).contiguous()
    tv = torch.from_numpy(vv)[None, None].expand(1, 4, 100, HD).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# Visible-row start, logit soft-cap and learned sinks ([P2] attend_group_upto)
# ---------------------------------------------------------------------------
def sdpa_bias(q, k, v, bias):
    """torch SDPA in float64 with an additive score bias [hpk][n] (-inf masks
    a row); k, v [n][hd] shared by the hpk query heads."""
    hpk, hd = q.shape
    n = k.shape[0]
    tq = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    tk = torch.from_numpy(np.asarray(k, np.float64))[None, None].expand(1, hpk, n, hd).contiguous()
    tv = torch.from_numpy(np.asarray(v, np.float64))[None, None].expand(1, hpk, n, hd).contiguous()
    tb = torch.from_numpy(np.asarray(bias, np.float64))[None, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tb)[0, :, 0, :].numpy()


def options_reference(q, k, v, first, softcap, sinks):
    """The options through torch: rows before the (clamped) first are masked
    with -inf, the cap enters as the bias cap*tanh(s/cap) - s on torch's own
    scaled scores, and a sink is one extra key row of zeros (score 0) with a
    zero value row and bias = the sink logit."""
    hpk, hd = q.shape
    n = k.shape[0]
    f = min(max(first, 0), n - 1)
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) / math.sqrt(hd)
    bias = np.zeros((hpk, n))
    if softcap > 0:
        bias = softcap * np.tanh(s / softcap) - s
    bias[:, :f] = -np.inf
    if sinks is None:
        return sdpa_bias(q, k, v, bias)
    k2 = np.concatenate([np.asarray(k, np.float64), np.zeros((1, hd))])
    v2 = np.concatenate([np.asarray(v, np.float64), np.zeros((1, hd))])
    bias2 = np.concatenate([bias, np.asarray(sinks, np.float64).reshape(hpk, 1)], axis=1)
    return sdpa_bias(q, k2, v2, bias2)


@pytest.mark.parametrize("n,first", [(1, 0), (9, 0), (9, 1), (9, 8), (9, 9), (9, 40), (300, 217)])
def test_window_equals_masked_rows(n, first):
    """[P2] attend_group_upto: only rows [first, stored) are scored, first is
    clamped to stored - 1, and the result equals the softmax over the whole
    row with -inf before first (page test windowed_attend_equals_masked_full_row)."""
    r = rng(3000 + n + first)
    q = r.standard_normal((3, HD)).astype(np.float32)
    k = (r.standard_normal((n, HD)) * 2).astype(np.float32)
    v = r.standard_normal((n, HD)).astype(np.float32)
    got = oracle.attend_f32(q, k, v, first=first)
    np.testing.assert_allclose(got, options_reference(q, k, v, first, 0.0, None), rtol=0, atol=1e-12)
    if first >= n:                                    # one visible row: its value, exactly
        assert np.array_equal(got, np.repeat(v[n - 1:n].astype(np.float64), 3, axis=0))


@pytest.mark.parametrize("cap", [0.5, 4.0, 30.0])
def test_softcap_matches_sdpa_with_tanh_bias(cap):
    """[P2] attend_group_upto, Gemma-2 soft-capping of the scaled scores."""
    r = rng(3100 + int(cap * 10))
    q = (r.standard_normal((4, HD)) * 3).astype(np.float32)
    k = (r.standard_normal((50, HD)) * 3).astype(np.float32)
    v = r.standard_normal((50, HD)).astype(np.float32)
    got = oracle.attend_f32(q, k, v, softcap=cap)
    np.testing.assert_allclose(got, options_reference(q, k, v, 0, cap, None), rtol=0, atol=1e-12)


def test_softcap_closed_forms():
    """Two keys: weights 1 : exp(c tanh(s2/c) - c tanh(s1/c)); a huge cap is
    no cap; a tiny cap squeezes every score into (-c, c), so the output tends
    to the mean of the values."""
    hd = 4
    q = np.array([1.0, 0.0, 0.0, 0.0], np.float32)
    k = np.array([[2.0, 0, 0, 0], [8.0, 0, 0, 0]], np.float32)          # scores 1 and 4
    v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]], np.float32)
    c = 2.0
    a = math.exp(c * math.tanh(1.0 / c))
    b = math.exp(c * math.tanh(4.0 / c))
    got = oracle.attend_f32(q, k, v, softcap=c)
    np.testing.assert_allclose(got[:2], [a / (a + b), b / (a + b)], rtol=0, atol=1e-15)
    r = rng(3200)
    q2 = r.standard_normal((2, HD)).astype(np.float32)
    k2 = r.standard_normal((30, HD)).astype(np.float32)
    v2 = r.standard_normal((30, HD)).astype(np.float32)
    np.testing.assert_allclose(oracle.attend_f32(q2, k2, v2, softcap=1e12), oracle.attend_f32(q2, k2, v2),
                               rtol=0, atol=1e-12)
    tiny = oracle.attend_f32(q2, k2, v2, softcap=1e-9)
    np.testing.assert_allclose(tiny, np.repeat(v2.astype(np.float64).mean(0)[None], 2, 0), rtol=0, atol=1e-7)


def test_sinks_match_value_less_column():
    """[P2] attend_group_upto: a sink logit takes part in the maximum and the
    normaliser and carries no value -- a softmax over the rows plus one extra column of
    value zero."""
    r = rng(3300)
    q = r.standard_normal((4, HD)).astype(np.float32)
    k = (r.standard_normal((40, HD)) * 2).astype(np.float32)
    v = r.standard_normal((40, HD)).astype(np.float32)
    z = np.array([0.5, -3.0, 9.0, 2.0], np.float32)
    got = oracle.attend_f32(q, k, v, sinks=z)
    np.testing.assert_allclose(got, options_reference(q, k, v, 0, 0.0, z), rtol=0, atol=1e-12)
    # a very negative sink takes no mass; a dominant one takes nearly all of it
    np.testing.assert_allclose(oracle.attend_f32(q, k, v, sinks=np.full(4, -1e4, np.float32)),
                               oracle.attend_f32(q, k, v), rtol=0, atol=0)
    one = oracle.attend_f32(q[:1], k[:1], v[:1], sinks=np.array([0.0], np.float32))
    s = float(q[0].astype(np.float64) @ k[0].astype(np.float64)) / math.sqrt(HD)
    w = math.exp(s) / (math.exp(s) + 1.0)                 # one row and a sink at 0
    np.testing.assert_allclose(one[0], w * v[0].astype(np.float64), rtol=0, atol=1e-15)


def test_sinks_with_windows_page_example():
    """[P2] test sink_attend_matches_explicit_sink_column: 2 KV heads x 8
    channels, 3 Q heads per group, 9 rows of the page's modular pattern, sinks
    (0.7, -1.3, 2.5, 0, -4, 6), prefixes of 1, 2, 5, 9 rows and windows of
    all, 3 and 1 rows; the page checks against an explicit value-less sink
    column computed in f64."""
    nkv, hd, hpk, rows = 2, 8, 3, 9

    def kv(r_, i, a, m):
        return np.float32((((r_ * a + i * 7 + 3) % m) / m - 0.5) * 2.0)

    K = np.array([[kv(r_, i, 31, 97) for i in range(nkv * hd)] for r_ in range(rows)], np.float32)
    V = np.array([[kv(r_, i, 17, 89) for i in range(nkv * hd)] for r_ in range(rows)], np.float32)
    q = np.array([(((i * 11 + 5) % 83) / 83.0 - 0.5) * 3.0 for i in range(nkv * hpk * hd)], np.float32)
    sinks = np.array([0.7, -1.3, 2.5, 0.0, -4.0, 6.0], np.float32)
    checked = 0
    for upto in (1, 2, 5, 9):
        for window in (None, 3, 1):
            first = 0 if window is None else max(upto - window, 0)
            for g in range(nkv):
                qg = q[g * hpk * hd:(g + 1) * hpk * hd].reshape(hpk, hd)
                kg, vg = K[:upto, g * hd:(g + 1) * hd], V[:upto, g * hd:(g + 1) * hd]
                zg = sinks[g * hpk:(g + 1) * hpk]
                got = oracle.attend_f32(qg, kg, vg, first=first, sinks=zg)
                np.testing.assert_allclose(got, options_reference(qg, kg, vg, first, 0.0, zg), rtol=0, atol=1e-12)
                checked += hpk
    assert checked == 4 * 3 * nkv * hpk


def test_all_options_on_q8_rows():
    """Window + soft-cap + sinks on a q8 head: the same options over the
    dequantised rows."""
    r = rng(3400)
    h = oracle.Q8Head(cap=200)
    h.append((r.standard_normal((200, HD)) * 3).astype(np.float32),
             (r.standard_normal((200, HD)) * 3).astype(np.float32))
    q = r.standard_normal((4, HD)).astype(np.float32)
    z = np.array([1.0, -2.0, 0.0, 5.0], np.float32)
    got = oracle.attend_q8(q, h, first=70, softcap=20.0, sinks=z)
    ref = options_reference(q, h.dequant_k(), h.dequant_v(), 70, 20.0, z)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_batched_driver_routes_first_and_sinks_per_sequence_and_head():
    """[P1] attend_group / [P2] attend_group_upto through the batched driver:
    Q head h reads KV head h // hpk, sequence b's first visible row is its own
    (clamped to its last row), and the sink logit of Q head h is sinks[h];
    each (b, h) against torch SDPA in f64 with the masked rows and the sink
    column written out, and dead groups give zeros."""
    r = rng(3500)
    B, hkv, hpk = 3, 3, 2
    hq = hkv * hpk
    lens = [37, 9, 20]
    first = [5, 40, 19]                               # inside, past the end (clamped to 8), the last row
    sinks = np.array([0.8, -2.5, 3.0, 0.1, -1.0, 4.5], np.float32)
    units = [[None] * hkv for _ in range(B)]
    for b, n in enumerate(lens):
        for g in range(hkv):
            if (b, g) == (1, 2):
                continue                              # a dead group
            units[b][g] = ("f32", (r.standard_normal((n, HD)) * 2).astype(np.float32),
                           r.standard_normal((n, HD)).astype(np.float32))
    q = r.standard_normal((B, hq, HD)).astype(np.float32)
    got = oracle.decode(q, units, hkv, first=first, sinks=sinks)
    for b in range(B):
        for g in range(hkv):
            sl = slice(g * hpk, (g + 1) * hpk)
            if units[b][g] is None:
                assert not got[b, sl].any()
                continue
            _, k, v = units[b][g]
            ref = options_reference(q[b, sl], k, v, first[b], 0.0, sinks[sl])
            np.testing.assert_allclose(got[b, sl], ref, rtol=0, atol=1e-12)
    plain = oracle.decode(q, units, hkv)
    for b in range(B):
        for g in range(hkv):
            if units[b][g] is not None:
                sl = slice(g * hpk, (g + 1) * hpk)
                np.testing.assert_allclose(plain[b, sl], options_reference(q[b, sl], units[b][g][1], units[b][g][2],
                                                                           0, 0.0, None), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# R-SWA ring cursors
# ---------------------------------------------------------------------------
def test_ring_slots_from_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ring_slots.json")))
    W = g["window"]
    m = oracle.RingModel(W)
    m.record_prefill(4)
    for t in range(W):
        assert m.write(t) == t and m.ring_len == t + 1 and m.effective_len() == 4 + t + 1
    assert m.ring_len == g["warmup"]["ring_len_after"] and m.ring_pos == g["warmup"]["ring_pos_after"]
    for slot, pos in zip(g["steady"]["slots"], g["steady"]["ring_pos_after_each"]):
        assert m.write("x") == slot and m.ring_pos == pos and m.ring_len == W
    m2 = oracle.RingModel(W)
    m2.record_prefill(1)
    for t in range(W):
        m2.write(t)
    for s in range(W):
        assert m2.write(W + s) == s
    assert m2.ring_pos == g["wrap"]["ring_pos_after"]
    for n, key in ((165, "writes_165_ring_pos"), (500, "writes_500_ring_pos")):
        m3 = oracle.RingModel(W)
        m3.record_prefill(0)
        for t in range(n):
            m3.write(t)
        assert m3.ring_pos == g["workload_cursors"][key] == n % W


def test_ring_physical_slots_closed_form():
    """After n writes token t sits in slot t mod W for every live t, and the
    live set is exactly the last min(n, W) tokens."""
    W = 128
    for n in (1, 5, 127, 128, 129, 300, 500):
        m = oracle.RingModel(W)
        m.record_prefill(3)
        for t in range(n):
            m.write(t)
        phys = m.physical()
        assert len(phys) == min(n, W)
        for t in range(max(0, n - W), n):
            assert phys[t % W] == t
        assert sorted(phys) == m.window() == list(range(max(0, n - W), n))


def test_ring_attention_equals_explicit_window():
    """Attention over reference rows ++ physical ring slots equals attention
    over reference rows ++ the explicit window of the last W tokens."""
    r = rng(19)
    W, prefill, n = 16, 5, 41
    ref_k = r.standard_normal((prefill, HD)).astype(np.float32)
    ref_v = r.standard_normal((prefill, HD)).astype(np.float32)
    tok_k = r.standard_normal((n, HD)).astype(np.float32)
    tok_v = r.standard_normal((n, HD)).astype(np.float32)
    m = oracle.RingModel(W)
    m.record_prefill(prefill)
    ring_k = np.zeros((W, HD), np.float32)
    ring_v = np.zeros((W, HD), np.float32)
    q = r.standard_normal((2, HD)).astype(np.float32)
    for t in range(n):
        s = m.write(t)
        ring_k[s], ring_v[s] = tok_k[t], tok_v[t]
        phys_k = np.concatenate([ref_k, ring_k[: m.ring_len]])
        phys_v = np.concatenate([ref_v, ring_v[: m.ring_len]])
        win = m.window()
        exp_k = np.concatenate([ref_k, tok_k[win]])
        exp_v = np.concatenate([ref_v, tok_v[win]])
        np.testing.assert_allclose(oracle.attend_f32(q, phys_k, phys_v),
                                   oracle.attend_f32(q, exp_k, exp_v), rtol=0, atol=1e-13)


def test_ring_rollback_restores_cursors_page_example():
    """[P3] tests checkpoint_rollback_restores_ring_rows_byte_identical and
    rollback_noop_is_identity: 5 prefill rows, 9 accepted steps, a checkpoint
    at ring_len = ring_pos = 9, 6 draft steps rolled back; the live window is
    the accepted tokens again and the next write lands in slot 9."""
    m = oracle.RingModel()
    m.record_prefill(5)
    for t in range(9):
        m.write(("acc", t))
    cp = m.checkpoint()
    assert (cp["ring_len"], cp["ring_pos"], cp["prefill_len"]) == (9, 9, 5)
    for t in range(6):
        m.write(("draft", t))
    assert m.ring_len == 15
    m.rollback_to(cp)
    assert (m.ring_len, m.ring_pos, m.writes, m.effective_len()) == (9, 9, 9, 14)
    assert m.physical() == [("acc", t) for t in range(9)] == m.window()
    assert m.slots[9] == ("draft", 0)                 # a dead slot keeps the discarded row
    assert m.write(("acc", 9)) == 9
    m2 = oracle.RingModel()
    m2.record_prefill(4)
    m2.write("a")
    e0 = m2.epoch
    m2.rollback_to(m2.checkpoint())                  # no-op rollback: identity, same lineage
    assert (m2.ring_len, m2.ring_pos, m2.writes, m2.epoch) == (1, 1, 1, e0)


def test_ring_rollback_refusals_page_examples():
    """[P3] tests rollback_rejects_eviction_in_steady_state_without_mutation
    and rollback_rejects_abandoned_branch_checkpoint_without_mutation, plus a
    checkpoint from the future and one from before a re-prefill."""
    m = oracle.RingModel()
    m.record_prefill(3)
    for _ in range(oracle.RING_W):
        m.write("x")
    cp = m.checkpoint()
    m.write("y")                                     # steady state: overwrites slot 0
    before = m.checkpoint()
    with pytest.raises(ValueError):
        m.rollback_to(cp)
    assert m.checkpoint() == before
    m = oracle.RingModel()
    m.record_prefill(4)
    m.write("accepted")
    branch = m.checkpoint()
    m.write("abandoned")
    stale = m.checkpoint()
    m.rollback_to(branch)
    m.write("replacement")
    assert (stale["ring_len"], stale["ring_pos"], stale["writes"]) == (m.ring_len, m.ring_pos, m.writes)
    before = m.checkpoint()
    with pytest.raises(ValueError):                  # same cursors, abandoned lineage
        m.rollback_to(stale)
    assert m.checkpoint() == before
    future = dict(before, writes=before["writes"] + 1)
    with pytest.raises(ValueError):
        m.rollback_to(future)
    old = m.checkpoint()
    m.record_prefill(4)                              # a re-prefill starts a new lineage
    with pytest.raises(ValueError):
        m.rollback_to(old)
    # a warm-up rollback may discard up to W - ring_len writes, no more
    m = oracle.RingModel()
    m.record_prefill(0)
    for _ in range(100):
        m.write(0)
    cp = m.checkpoint()
    for _ in range(oracle.RING_W - 100):
        m.write(1)
    m.rollback_to(cp)
    for _ in range(oracle.RING_W - 99):
        m.write(1)
    with pytest.raises(ValueError):
        m.rollback_to(cp)


def test_ring_reprefill_resets_cursors():
    """[P3] RingCache::record_prefill: a new prefill empties the ring -- length,
    position and write count back to 0 -- so the effective length is the new
    reference length and the next write lands in slot 0, from steady state
    as from warm-up."""
    for writes in (7, oracle.RING_W + 37):
        m = oracle.RingModel()
        m.record_prefill(11)
        for t in range(writes):
            m.write(t)
        m.record_prefill(23)
        assert (m.prefill_len, m.ring_len, m.ring_pos, m.writes) == (23, 0, 0, 0)
        assert m.window() == [] and m.physical() == [] and m.effective_len() == 23
        assert m.write("new") == 0 and m.window() == ["new"] and m.effective_len() == 24


def test_trim_window_page_invariants():
    """[P2] tests swa_trim_keeps_contiguous_tail and swa_gen_bumps: feeding
    positions one by one with w = 6, slack 2, align 4, a trim leaves
    w + slack .. w + slack + align - 1 rows, never more than 2w rows stay,
    the base stays a multiple of align and base + rows is the position
    count; with w = 10, 18 rows do not trim and 21 do."""
    w, slack, align = 6, 2, 4
    base, n, trims = 0, 0, 0
    for p in range(100):
        n += 1
        d = oracle.trim_window(base, n, w, slack, align)
        if d:
            trims += 1
            base, n = base + d, n - d
            assert w + slack <= n < w + slack + align
        assert n <= 2 * w and base % align == 0 and base + n == p + 1
    assert trims > 5
    assert oracle.trim_window(0, 18, 10, 2, 4) == 0
    assert oracle.trim_window(0, 21, 10, 2, 4) > 0
    assert oracle.trim_window(0, 500, 0, 2, 4) == 0                     # w = 0: never
    assert oracle.trim_window(0, 500, 10, 2, 4, q8_unfrozen=True) == 0   # q8 field not frozen yet


def test_trim_window_page_bounds_sweep():
    """[P2] LayerKvCache::trim_window (doc and body): with at most 2w rows
    stored nothing is dropped; past that the front is drained down to
    w + slack rows, the cut rounded down to an absolute position that is a
    multiple of align, so that w + slack .. w + slack + align - 1 rows stay
    (nothing is dropped when the rounded cut does not pass the base).  Swept
    over w, slack, align, base and length; align 1 leaves exactly w + slack
    rows."""
    for w in (1, 3, 10, 64):
        for slack in (0, 1, 5):
            for align in (1, 2, 4, 16):
                for base in (0, 3, 37, 64):
                    assert oracle.trim_window(base, 2 * w, w, slack, align) == 0
                    for n in (2 * w + 1, 2 * w + 7, 5 * w + 3, 1000):
                        d = oracle.trim_window(base, n, w, slack, align)
                        cut = (base + n - (w + slack)) // align * align
                        if cut <= base:
                            assert d == 0, (w, slack, align, base, n, d)
                            continue
                        stay = n - d
                        assert (base + d) % align == 0, (w, slack, align, base, n, d)
                        assert w + slack <= stay <= w + slack + align - 1, (w, slack, align, base, n, d)
                        if align == 1:
                            assert stay == w + slack


def test_trim_window_anchored_page_example():
    """[P2] test swa_anchored_trim_keeps_the_rollback_window: with anchor 40
    (w 6, slack 2, align 4) the base never passes anchor - slack + 1 - w, so
    truncating back to anchor - slack leaves at least w - 1 rows; the plain
    trim then drains again."""
    w, slack, align, anchor = 6, 2, 4, 40
    base, n = 0, 0
    for p in range(100):
        n += 1
        d = oracle.trim_window(base, n, w, slack, align, anchor)
        base, n = base + d, n - d
        assert base + w <= anchor - slack + 1
    back = anchor - slack
    n = oracle.truncate_last(n, base + n - back)
    assert base + n == back and n >= w - 1
    for p in range(back, back + 3 * w):
        n += 1
        d = oracle.trim_window(base, n, w, slack, align)
        base, n = base + d, n - d
    assert n <= 2 * w
    assert oracle.truncate_last(5, 7) == 0 and oracle.truncate_last(5, 2) == 3


def test_head_truncate_page_examples():
    """[P2] truncate_last on the per-head stores: the page's q8 test appends
    100 positions (crossing the freeze) and truncates 30, leaving 70 rows;
    its f32 test keeps positions 0..2 of 5 after dropping 2.  The kept rows
    keep their codes and scales, and the frozen field stays."""
    r = rng(4100)
    k = (r.standard_normal((100, HD)) * 3).astype(np.float32)
    v = (r.standard_normal((100, HD)) * 3).astype(np.float32)
    h = oracle.Q8Head(cap=100)
    h.append(k, v)
    kq, ks, vq, vs = h.kq.copy(), h.ks.copy(), h.vq.copy(), h.vs.copy()
    kcol, vcol = h.kcol.copy(), h.vcol.copy()
    h.truncate_last(30)
    assert h.n == 70 and h.frozen
    assert np.array_equal(h.kq[:70], kq[:70]) and np.array_equal(h.vq[:70], vq[:70])
    assert np.array_equal(h.ks[:70], ks[:70]) and np.array_equal(h.vs[:70], vs[:70])
    assert np.array_equal(h.kcol, kcol) and np.array_equal(h.vcol, vcol)
    np.testing.assert_array_equal(h.dequant_k(), oracle.Q8Head.dequant_k(h)[:70])
    h.truncate_last(500)
    assert h.n == 0 and h.frozen
    i = oracle.I8Head(cap=5)
    rows = np.repeat(np.arange(5, dtype=np.float32)[:, None], HD, 1)
    i.append(rows, rows)
    i.truncate_last(2)
    assert i.n == 3
    # position 2 survives: a constant row of 2 codes as 127 x (2 / 127)
    assert (i.kq[2] == 127).all() and i.ks[2] == np.float32(2.0) / np.float32(127.0)
    np.testing.assert_allclose(i.dequant_k()[2], 2.0, rtol=1e-6)


@pytest.mark.parametrize("n0,nd", [(50, 10), (150, 20)])
def test_head_truncate_then_append_equals_never_appended(n0, nd):
    """A speculative append, truncated, then the accepted rows: the stores
    equal a head that only ever saw the accepted rows -- for q8 both when
    the rejected rows stay below the freeze (the freeze then happens at the
    same row) and after it (the rejected rows were quantised against the
    frozen field, which stays)."""
    r = rng(4200 + n0)
    base = [(r.standard_normal((n0, HD)) * 2).astype(np.float32) for _ in range(2)]
    draft = [(r.standard_normal((nd, HD)) * 5).astype(np.float32) for _ in range(2)]
    final = [(r.standard_normal((30, HD)) * 2).astype(np.float32) for _ in range(2)]
    for cls in (oracle.Q8Head, oracle.I8Head):
        t, c = cls(cap=300), cls(cap=300)
        t.append(*base)
        t.append(*draft)
        t.truncate_last(nd)
        c.append(*base)
        for h in (t, c):
            h.append(*final)
        assert t.n == c.n == n0 + 30
        for nm in ("kq", "ks", "vq", "vs"):
            assert np.array_equal(getattr(t, nm)[: t.n], getattr(c, nm)[: c.n]), (cls.__name__, nm)
        if cls is oracle.Q8Head:
            assert t.frozen and c.frozen
            assert np.array_equal(t.kcol, c.kcol) and np.array_equal(t.vcol, c.vcol)


def test_q8_truncate_below_warmup_keeps_the_frozen_field():
    """[P2] truncate_last drops rows only: a head frozen at 64 and truncated
    to 10 rows quantises its next row against the frozen field (reading
    c32), not against a field of 1."""
    r = rng(4300)
    k = (r.standard_normal((80, HD)) * np.exp(r.uniform(-1, 2, HD))).astype(np.float32)
    v = (r.standard_normal((80, HD)) * np.exp(r.uniform(-1, 2, HD))).astype(np.float32)
    h = oracle.Q8Head(cap=100)
    h.append(k, v)
    h.truncate_last(70)
    assert h.n == 10 and h.frozen
    x = (r.standard_normal((1, HD)) * 4).astype(np.float32)
    h.append(x, x)
    kq, ks = oracle.quant_row(x[0], h.kcol)
    vq, vs = oracle.quant_row(x[0], h.vcol, group=HD)
    assert np.array_equal(h.kq[10], kq) and np.array_equal(h.ks[10], ks)
    assert np.array_equal(h.vq[10], vq) and h.vs[10] == vs[0]
    k1, _ = oracle.quant_row(x[0])
    assert not np.array_equal(kq, k1)


@pytest.mark.parametrize("prefill,n_hist,K", [(7, 5, 4), (7, 126, 5), (3, 300, 6), (0, 0, 3)])
def test_verify_equals_sequential_ring_steps(prefill, n_hist, K):
    """[P3] verify_attention: draft i's context is the i-th of K sequential
    decode steps -- computed here on the physical ring of a RingModel
    (pinned by the ring tests), written slot by slot, warm-up, crossing the
    window and in steady state; query i never sees drafts after i."""
    r = rng(4000 + prefill + n_hist + K)
    hkv, hpk, W = 2, 2, oracle.RING_W
    ref_k = r.standard_normal((hkv, prefill, HD)).astype(np.float32)
    ref_v = r.standard_normal((hkv, prefill, HD)).astype(np.float32)
    hist_k = r.standard_normal((hkv, n_hist, HD)).astype(np.float32)
    hist_v = r.standard_normal((hkv, n_hist, HD)).astype(np.float32)
    dk = r.standard_normal((K, hkv, HD)).astype(np.float32)
    dv = r.standard_normal((K, hkv, HD)).astype(np.float32)
    q = r.standard_normal((K, hkv * hpk, HD)).astype(np.float32)
    got = oracle.rswa_verify(q, ref_k, ref_v, hist_k, hist_v, dk, dv)
    m = oracle.RingModel(W)
    m.record_prefill(prefill)
    ring_k = np.zeros((hkv, W, HD), np.float32)
    ring_v = np.zeros((hkv, W, HD), np.float32)
    for t in range(n_hist):
        s_ = m.write(t)
        ring_k[:, s_], ring_v[:, s_] = hist_k[:, t], hist_v[:, t]
    for i in range(K):
        s_ = m.write(n_hist + i)
        ring_k[:, s_], ring_v[:, s_] = dk[i], dv[i]
        for g in range(hkv):
            rows_k = np.concatenate([ref_k[g], ring_k[g, : m.ring_len]])
            rows_v = np.concatenate([ref_v[g], ring_v[g, : m.ring_len]])
            want = oracle.attend_f32(q[i, g * hpk:(g + 1) * hpk], rows_k, rows_v)
            np.testing.assert_allclose(got[i, g * hpk:(g + 1) * hpk], want, rtol=0, atol=1e-13)
    # a later draft token does not reach an earlier query
    dk2, dv2 = dk.copy(), dv.copy()
    dk2[-1] += 5.0
    dv2[-1] -= 3.0
    got2 = oracle.rswa_verify(q, ref_k, ref_v, hist_k, hist_v, dk2, dv2)
    assert np.array_equal(got2[:-1], got[:-1]) and not np.array_equal(got2[-1], got[-1])


@pytest.mark.parametrize("prefill,n_hist,K", [(7, 5, 4), (7, 126, 5), (3, 300, 6), (0, 0, 3)])
def test_verify_i8_equals_sequential_int8_decodes(prefill, n_hist, K):
    """The verify on the int8 mirror: draft i's context is the i-th of K
    sequential steps on the mirror -- each row quantised once as it is
    written (quantize_row_i8, a row's codes do not depend on the others) and
    decode_attention_int8 over the physical ring of a RingModel."""
    r = rng(4100 + prefill + n_hist + K)
    hkv, hpk, W = 2, 2, oracle.RING_W
    ref_k = (r.standard_normal((hkv, prefill, HD)) * 2).astype(np.float32)
    ref_v = r.standard_normal((hkv, prefill, HD)).astype(np.float32)
    hist_k = (r.standard_normal((hkv, n_hist, HD)) * 2).astype(np.float32)
    hist_v = r.standard_normal((hkv, n_hist, HD)).astype(np.float32)
    dk = (r.standard_normal((K, hkv, HD)) * 2).astype(np.float32)
    dv = r.standard_normal((K, hkv, HD)).astype(np.float32)
    q = r.standard_normal((K, hkv * hpk, HD)).astype(np.float32)
    got = oracle.rswa_verify(q, ref_k, ref_v, hist_k, hist_v, dk, dv, kind="i8")
    m = oracle.RingModel(W)
    m.record_prefill(prefill)
    codes = {g: {} for g in range(hkv)}               # slot -> (kq, ks, vq, vs)
    for t in range(n_hist + K):
        s_ = m.write(t)
        for g in range(hkv):
            kx = hist_k[g, t] if t < n_hist else dk[t - n_hist, g]
            vx = hist_v[g, t] if t < n_hist else dv[t - n_hist, g]
            codes[g][s_] = oracle.quant_row_i8(kx) + oracle.quant_row_i8(vx)
        if t < n_hist:
            continue
        i = t - n_hist
        for g in range(hkv):
            h = oracle.I8Head(cap=prefill + m.ring_len + 1)
            if prefill:
                h.append(ref_k[g], ref_v[g])
            for slot in range(m.ring_len):
                kq, ks, vq, vs = codes[g][slot]
                h.kq[h.n], h.ks[h.n], h.vq[h.n], h.vs[h.n] = kq, ks, vq, vs
                h.n += 1
            want = oracle.attend_i8(q[i, g * hpk:(g + 1) * hpk], h)
            np.testing.assert_allclose(got[i, g * hpk:(g + 1) * hpk], want, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Per-row int8 route ([P3] quantize_row_i8, decode_attention_int8)
# ---------------------------------------------------------------------------
def test_int8_row_fixtures_from_page(golden_dir):
    """[P3] tests: ties to even ([127, .5, 1.5, ...] -> [127, 0, 2, 2, 4, 0,
    -2, -2, -4], scale 1) and division, not the reciprocal (-124, where
    the reciprocal route gives -125)."""
    fx = json.load(open(os.path.join(golden_dir, "int8_row_fixtures.json")))
    row = np.zeros(HD, np.float32)
    row[:9] = fx["ties_to_even"]["row_prefix"]
    q, sc = oracle.quant_row_i8(row)
    assert q[:9].tolist() == fx["ties_to_even"]["codes_prefix"] and not q[9:].any()
    assert struct.pack("<f", sc).hex() == struct.pack("<I", int(fx["ties_to_even"]["scale_bits"], 16)).hex()
    row = np.zeros(HD, np.float32)
    row[:2] = [bits_f32(h) for h in fx["divides"]["row_prefix_bits"]]
    q, sc = oracle.quant_row_i8(row)
    assert q[:2].tolist() == fx["divides"]["codes_prefix"]
    recip = half_away(float(np.float32(row[1] * np.float32(np.float32(1.0) / sc))))
    assert recip == fx["divides"]["reciprocal_route_code_1"]


def test_int8_row_against_exact_rationals():
    """scale = f32(maxabs / 127) and code = round_ties_even(f32(x / scale))
    recomputed with exact rationals over rows of magnitudes 2^-20 .. 2^20
    (the page's scalar-contract test spans the same range); an all-zero row
    has scale 1 and codes 0."""
    r = rng(5000)
    for case in range(60):
        mag = 2.0 ** ((case % 41) - 20)
        x = ((r.random(HD) * 2 - 1) * mag).astype(np.float32)
        if case == 0:
            x[:] = 0
        q, sc = oracle.quant_row_i8(x)
        amax = max(abs(Fraction(float(v))) for v in x)
        want_sc = f32_round(amax / 127) if amax > 0 else 1.0
        assert float(sc) == want_sc
        for d in range(HD):
            t = f32_round(Fraction(float(x[d])) / Fraction(want_sc))
            want = max(-127, min(127, round(t)))          # Python rounds ties to even
            assert q[d] == want, (case, d)


def test_int8_attention_matches_sdpa_on_dequantised_rows():
    """decode_attention_int8 is attention of the dequantised query q^ =
    code * qscale over K^ = code * kscale, V^ = code * vscale (torch SDPA,
    float64)."""
    r = rng(5100)
    h = oracle.I8Head(cap=90)
    h.append((r.standard_normal((90, HD)) * 3).astype(np.float32),
             (r.standard_normal((90, HD)) * 3).astype(np.float32))
    q = (r.standard_normal((4, HD)) * 2).astype(np.float32)
    got = oracle.attend_i8(q, h)
    qh = np.stack([oracle.quant_row_i8(q[i])[0].astype(np.float64) * float(oracle.quant_row_i8(q[i])[1])
                   for i in range(4)])
    tq = torch.from_numpy(qh)[None, :, None, :]
    tk = torch.from_numpy(h.dequant_k())[None, None].expand(1, 4, 90, HD).contiguous()
    tv = torch.from_numpy(h.dequant_v())[None, None].expand(1, 4, 90, HD).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    # the integer dot stays far inside i32: 127 * 127 * 128
    assert 127 * 127 * HD == 2_064_512 < 2 ** 31


@pytest.mark.parametrize("first,with_sinks", [(0, True), (37, False), (37, True), (89, True), (500, False)])
def test_int8_attention_options_match_sdpa(first, with_sinks):
    """The visible-row start and value-less sink logits on the int8 route
    equal the same options ([P2] attend_group_upto) on the dequantised query
    and rows: torch SDPA in float64 with -inf before the clamped first row and
    a zero key/value column biased by the sink."""
    r = rng(5200 + first + 7 * with_sinks)
    h = oracle.I8Head(cap=90)
    h.append((r.standard_normal((90, HD)) * 3).astype(np.float32),
             (r.standard_normal((90, HD)) * 3).astype(np.float32))
    q = (r.standard_normal((4, HD)) * 2).astype(np.float32)
    z = (r.standard_normal(4) * 4).astype(np.float32) if with_sinks else None
    got = oracle.attend_i8(q, h, first=first, sinks=z)
    qh = np.stack([oracle.quant_row_i8(q[i])[0].astype(np.float64) * float(oracle.quant_row_i8(q[i])[1])
                   for i in range(4)])
    ref = options_reference(qh, h.dequant_k(), h.dequant_v(), first, 0.0, z)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_workload_generators_are_deterministic():
    s = workloads.get("batched_q8")
    L = s.lengths()
    assert L.min() >= 1024 and L.max() <= 32768 and len(L) == 64
    k1, v1 = s.kv_rows(3, 10, 5)
    k2, v2 = s.kv_rows(3, 0, 15)
    assert np.array_equal(k1, k2[10:]) and np.array_equal(v1, v2[10:])
    fk, fv = s.factors(3)
    assert fk.min() >= 0.25 and fk.max() <= 8.0 and not np.array_equal(fk, fv)
