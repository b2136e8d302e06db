"""Plants plausible mistakes in a COPY of the oracle source (CPU only) and
checks that the oracle pins catch every one of them.

Each C mutant is a one-line edit of oracle/kvq_oracle.c, compiled into a
temporary library that a child pytest process loads in place of the real
oracle; each Python mutant is an edit of a copy of oracle/__init__.py (the
ring cursor model, rollback, the verify, the batch driver's GQA mapping,
truncate and the trim) that the child process imports in place of the real
package.  The pin suite must fail for every one.  (A lower clamp of -128 is not listed:
|r/s| never rounds beyond 127, so that edit cannot change any output.)
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvq_oracle.c")

MUTANTS = {
    "round_ties_even": ("float r = roundf(resid[d] / sc);", "float r = rintf(resid[d] / sc);"),
    "reciprocal": ("float r = roundf(resid[d] / sc);", "float r = roundf(resid[d] * (1.0f / sc));"),
    "col_multiplies": ("x[d] / col[d]", "x[d] * col[d]"),
    "no_scale_floor": ("if (sc < 1e-12f) sc = 1e-12f;", ""),
    "scale_1_over_hd": ("double scale = 1.0 / sqrt((double)hd);\n    double* s",
                        "double scale = 1.0 / (double)hd;\n    double* s"),
    "softmax_no_max": ("s[p] = exp(s[p] - m); z += s[p];", "s[p] = exp(s[p]); z += s[p];"),
    "transposed_v": ("oh[d] += w * vf(vctx, p, d);", "oh[d] += w * vf(vctx, d % n, p % hd);"),
    "rms_no_mean": ("float c = sqrtf(col[d] / (float)n);", "float c = sqrtf(col[d]);"),
    "rms_wrong_n": ("float c = sqrtf(col[d] / (float)n);", "float c = sqrtf(col[d] / (float)(n + 1));"),
    "freeze_one_late": ("if (*n >= ORC_COL_WARMUP && !*frozen)", "if (*n > ORC_COL_WARMUP && !*frozen)"),
    "dequant_drops_scale": ("(float)q[(size_t)p * hd + d] * s[(size_t)p * ns + d / group];",
                            "(float)q[(size_t)p * hd + d];"),
    "q8_drops_col": ("if (r->col != NULL) x = x * (double)r->col[d];", ""),
    "q8_wrong_group": ("* (double)r->scales[(size_t)p * r->ns + d / r->group];",
                       "* (double)r->scales[(size_t)p * r->ns + (d / r->group) % 2];"),
    "fused_rms": ("float sq = x * x;\n            col[d] = col[d] + sq;", "col[d] = fmaf(x, x, col[d]);"),
    "requant_wrong_row": ("orc_quant_row(rows + (size_t)p * hd, col", "orc_quant_row(rows + 0 * (size_t)p * hd, col"),
    "window_clamp_two_rows": ("if (first > n - 1) first = n - 1;", "if (first > n - 1) first = n - 2 < 0 ? 0 : n - 2;"),
    "sink_not_in_denominator": ("if (sinks != NULL) z += exp((double)sinks[h] - m);", ""),
    "sink_scaled": ("z += exp((double)sinks[h] - m);", "z += exp((double)sinks[h] * scale - m);"),
    "sink_capped": ("z += exp((double)sinks[h] - m);",
                    "z += exp((softcap > 0.0 ? softcap * tanh((double)sinks[h] / softcap) : (double)sinks[h]) - m);"),
    "i8_half_away": ("float r = rintf(x[d] / scale);", "float r = roundf(x[d] / scale);"),
    "i8_reciprocal": ("float r = rintf(x[d] / scale);", "float r = rintf(x[d] * (1.0f / scale));"),
    "i8_zero_row_scale": ("float scale = maxabs > 0.0f ? maxabs / 127.0f : 1.0f;",
                          "float scale = maxabs > 0.0f ? maxabs / 127.0f : 1e-12f;"),
    "i8_drops_vscale": ("double w = s[p] / z * (double)vs[p];", "double w = s[p] / z;"),
    "i8_drops_qscale": ("s[p] = (double)dot * (double)qs * (double)ks[p] * scale;",
                        "s[p] = (double)dot * (double)ks[p] * scale;"),
    "i8_first_ignored": ("if (first < 0) first = 0;\n    int8_t* qc", "first = 0;\n    int8_t* qc"),
    "i8_sink_not_in_denominator": ("if (sinks != NULL) z += exp((double)sinks[h] - m);", "", 2),
    "i8_sink_scaled": ("z += exp((double)sinks[h] - m);", "z += exp((double)sinks[h] * scale - m);", 2),
    "softcap_missing_factor": ("s[p] = softcap * tanh(s[p] / softcap);", "s[p] = tanh(s[p] / softcap);"),
    "softcap_before_scale": ("s[p] = dot * scale;\n            if (softcap > 0.0) s[p] = softcap * tanh(s[p] / softcap);",
                             "s[p] = dot;\n            if (softcap > 0.0) s[p] = softcap * tanh(s[p] / softcap);\n"
                             "            s[p] = s[p] * scale;"),
}

RUNNER = r'''
import sys
sys.path.insert(0, sys.argv[2])
import oracle
oracle._LIB = sys.argv[1]
oracle.build = lambda force=False: sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", sys.argv[3]]))
'''


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new, nth = (MUTANTS[name] + (1,))[:3]         # nth: which occurrence to edit
    assert src.count(old) >= nth, "mutation site not found: " + name
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    at = -1
    for _ in range(nth):
        at = src.index(old, at + 1)
    c.write_text(src[:at] + new + src[at + len(old):])
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(so), str(c), "-lm"], check=True)
    runner = tmp_path / "run.py"
    runner.write_text(RUNNER)
    pins = os.path.join(ROOT, "tests", "test_oracle_pins.py")
    r = subprocess.run([sys.executable, str(runner), str(so), ROOT, pins],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant survived the pins: " + name


# Mutants of the oracle's Python half (oracle/__init__.py): the R-SWA ring
# cursor model, checkpoint / rollback, the K-draft verify, the GQA mapping of
# the batch driver, truncate and the sliding-window trim.
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PY_MUTANTS = {
    "ring_steady_slot_ahead": ("            slot = self.ring_pos\n            self.ring_pos = (self.ring_pos + 1) % self.W",
                               "            slot = (self.ring_pos + 1) % self.W\n            self.ring_pos = (self.ring_pos + 1) % self.W"),
    "ring_pos_stuck": ("self.ring_pos = (self.ring_pos + 1) % self.W", "self.ring_pos = self.ring_pos % self.W"),
    "window_one_short": ("return self.tokens[-self.W:] if self.tokens else []",
                         "return self.tokens[-(self.W - 1):] if self.tokens else []"),
    "rollback_allows_eviction": ('discarded > self.W - cp["ring_len"]', 'discarded > self.W'),
    "rollback_keeps_lineage": ("        if discarded:\n            self.epoch += 1", "        pass"),
    "verify_sees_next_draft": ("toks_k = np.concatenate([history_k[g], draft_k[: i + 1, g]])",
                               "toks_k = np.concatenate([history_k[g], draft_k[: i + 2, g]])"),
    "verify_ring_one_long": ("rows_k = np.concatenate([ref_k[g], toks_k[-window:]])",
                             "rows_k = np.concatenate([ref_k[g], toks_k[-window - 1:]])"),
    "decode_wrong_group": ("qg = np.ascontiguousarray(q[b, g * hpk:(g + 1) * hpk])",
                           "qg = np.ascontiguousarray(q[b, g:g + hpk])"),
    "truncate_one_more": ("return n - min(n_drop, n)", "return max(n - n_drop - 1, 0)"),
    "trim_no_slack": ("keep_from = max(base + n - (w + slack), 0)", "keep_from = max(base + n - w, 0)"),
    "trim_trigger_strict": ("if w == 0 or n <= 2 * w or q8_unfrozen:", "if w == 0 or n < 2 * w or q8_unfrozen:"),
    "trim_align_up": ("new_base = keep_from // align * align", "new_base = -(-keep_from // align) * align"),
    "trim_anchor_ignored": ("        keep_from = min(keep_from, max(anchor - (w + slack), 0))", "        pass"),
    "decode_first_shifted": ("f = 0 if first is None else int(first[b])", "f = 0 if first is None else int(first[b]) + 1"),
    "decode_sinks_wrong_heads": ("np.asarray(sinks, np.float32)[g * hpk:(g + 1) * hpk]",
                                 "np.asarray(sinks, np.float32)[g:g + hpk]"),
    "rollback_from_future": ('if cp["writes"] > self.writes:', 'if cp["writes"] > self.writes + 1:'),
    "prefill_keeps_ring": ("        self.prefill_len = n\n        self.ring_len = 0",
                           "        self.prefill_len = n\n        self.ring_len = self.ring_len"),
}

PY_RUNNER = r'''
import sys
sys.path.insert(0, sys.argv[2])
sys.path.insert(0, sys.argv[1])
import oracle
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", sys.argv[3]]))
'''


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_catch_python_mutant(name, tmp_path):
    import shutil
    src = open(PY_SRC).read()
    old, new = PY_MUTANTS[name]
    assert src.count(old) == 1, "mutation site not found: " + name
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy2(os.path.join(ROOT, "oracle", "kvq_oracle.c"), pkg / "kvq_oracle.c")
    built = os.path.join(ROOT, "oracle", "libkvq_oracle.so")
    if os.path.exists(built):
        shutil.copy2(built, pkg / "libkvq_oracle.so")
    (pkg / "__init__.py").write_text(src.replace(old, new))
    runner = tmp_path / "run.py"
    runner.write_text(PY_RUNNER)
    pins = os.path.join(ROOT, "tests", "test_oracle_pins.py")
    r = subprocess.run([sys.executable, str(runner), str(tmp_path), ROOT, pins],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant survived the pins: " + name + "\n" + r.stdout[-2000:]
