"""Decode-attention benchmark on one MI355X.

One step = one decode step of the two 32k-context workloads, every part of
the hot path through the C ABI:
  * R-SWA long reference, f32: rswa_decode (ring write + split-K attention +
    combine) over 10 MHA heads x (32640 reference rows + a full 128-slot ring);
  * batched GQA q8_2f: kv_append_q8 of one new row per sequence (the
    quantiser; sequences crossing 64 rows would freeze), then decode_attn_q8
    over 64 sequences x 8 KV heads (32 Q heads), lengths uniform in
    [1024, 32768].
Inputs are seeded synthetic tensors already resident in HBM.  The f32
caches are rotated over replicas totalling >= 1 GB so the 256 MB Infinity
Cache cannot serve repeated reads; the q8 cache alone is ~2.3 GB.

Prints ONE JSON line: KV positions/s for the whole step, per-part GB/s and
fraction of the 8 TB/s HBM peak, the roofline of the dominant kernel (the
q8 decode) timed with HIP events on its own stream, and the CPU oracle timed
on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "decode-attn KV positions/s + achieved HBM GB/s (% of peak), f32 and q8"
HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--replicas", type=int, default=4, help="f32 R-SWA cache replicas (>= 1 GB total)")
    p.add_argument("--part", choices=["both", "rswa", "q8", "small"], default="both",
                   help="small: only the three small workloads' per-call timings (no step)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-small", action="store_true", help="skip the three small workloads")
    p.add_argument("--cpu-sample-seqs", type=int, default=8)
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="host time the oracle sample is repeated for")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 512 MiB device-to-device copy (for counter calibration)")
    return p.parse_args()


def calibrate_copy():
    """A plain device copy of known size: under rocprofv3 --pmc its FETCH_SIZE
    and WRITE_SIZE per dispatch give the counters' bytes-per-byte factors."""
    import torch
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "dispatches": 5}))


def algorithmic_bytes_q8(lens, n_live, hq):
    rows = int(np.sum(lens)) * n_live
    return rows * 276 + len(lens) * n_live * 2 * 128 * 4 + len(lens) * hq * 128 * 4 * 2


def algorithmic_bytes_i8(lens, n_live, hq):
    # int8 K and V codes (2 x 128 B) and their two f32 row scales per row
    # and live head, queries read, outputs written
    rows = int(np.sum(lens)) * n_live
    return rows * 264 + len(lens) * hq * 128 * 4 * 2


def algorithmic_bytes_rswa_i8(n_rows, heads):
    # int8 K/V rows and their row scales read once (264 B per row and head),
    # q read, out written, the step's f32 K/V read and its codes + scales written
    return n_rows * heads * 264 + heads * 512 * 2 + heads * (512 * 2 + 264)


def algorithmic_bytes_rswa(n_rows, heads):
    # K and V rows read once, q read, out written, the step's K/V read and written once
    return n_rows * heads * 1024 + heads * 512 * 2 + heads * 512 * 2 * 2


def source_digest():
    h = hashlib.sha256()
    for f in ("kvq_decode.hip", "kvq_internal.h"):
        h.update(open(os.path.join(ROOT, "int8_kv_cache_decode_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None when missing or taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, kernel_tag + "_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"source_digest:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from int8_kv_cache_decode_amd import kvq as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    do_rswa = args.part in ("both", "rswa")
    do_q8 = args.part in ("both", "q8")
    total_steps = args.warmup + args.steps
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    # ---------------- R-SWA long reference, f32 ----------------
    rs = workloads.get("rswa_long_f32")
    rswa = []
    if do_rswa:
        rk, rv = rs.reference()
        rk_d = t(rk.transpose(1, 0, 2))
        rv_d = t(rv.transpose(1, 0, 2))
        pool = [tuple(t(x[None]) for x in rs.step(s)) for s in range(16)]
        for rep in range(args.replicas):
            c = K.KvCache(K.KIND_F32, 1, rs.n_heads, rs.prefill + rs.window)
            rings = K.Rings(1)
            K.kv_append_f32(c, 0, rs.prefill, rk_d, rv_d)
            K.rswa_record_prefill(c, rings, 0)
            out = torch.zeros((1, rs.n_heads, 128), device=dev)
            for s in range(rs.writes - 1):          # reach the steady state (ring full)
                q, kk, vv = pool[s % 16]
                K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
            rswa.append((c, rings, out))
        # the same reference and steps on the int8 mirror ([P3] Int8Kv):
        # 86.5 MB per replica, 6 replicas so the MALL cannot serve repeats
        rswa_i8 = []
        for rep in range(6):
            c = K.KvCache(K.KIND_I8, 1, rs.n_heads, rs.prefill + rs.window)
            rings = K.Rings(1)
            K.kv_append_i8(c, 0, rs.prefill, rk_d, rv_d)
            K.rswa_record_prefill(c, rings, 0)
            out = torch.zeros((1, rs.n_heads, 128), device=dev)
            for s_ in range(rs.writes - 1):
                q, kk, vv = pool[s_ % 16]
                K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
            rswa_i8.append((c, rings, out))
        del rk_d, rv_d
        torch.cuda.synchronize()
        log("rswa replicas ready: %d x %.1f MB, ring_len %d ring_pos %d" % (
            args.replicas, rs.n_heads * (rs.prefill + rs.window) * 1024 / 1e6,
            rswa[0][1][0].ring_len, rswa[0][1][0].ring_pos))

    # ---------------- batched GQA q8_2f ----------------
    bq = workloads.get("batched_q8")
    lens = bq.lengths()
    if do_q8:
        from concurrent.futures import ThreadPoolExecutor
        cq = K.KvCache(K.KIND_Q8, bq.batch, bq.n_kv_heads, int(lens.max()) + total_steps + 64)
        # the same rows also go through the per-row int8 codec ([P3])
        ci8 = K.KvCache(K.KIND_I8, bq.batch, bq.n_kv_heads, int(lens.max()))
        with ThreadPoolExecutor(16) as ex:
            for b, (k, v) in enumerate(ex.map(bq.kv_rows, range(bq.batch))):
                kd, vd = t(k), t(v)
                K.kv_append_q8(cq, b, int(lens[b]), kd, vd)
                K.kv_append_i8(ci8, b, int(lens[b]), kd, vd)
        qq = t(bq.query())
        qout = torch.zeros((bq.batch, bq.n_q_heads, 128), device=dev)
        newk = t(workloads.normal_f32(workloads.key(bq.seed, 99), (bq.batch, bq.n_kv_heads, 128)))
        newv = t(workloads.normal_f32(workloads.key(bq.seed, 98), (bq.batch, bq.n_kv_heads, 128)))
        ws_q8 = cq.workspace(bq.n_q_heads)
        torch.cuda.synchronize()
        log("q8 cache ready: %d rows, %.2f GB stored (i8: %.2f GB)" % (
            int(lens.sum()), cq.cache_bytes() / 1e9, ci8.cache_bytes() / 1e9))

    # ---------------- per-part kernel timing with HIP events ----------------
    # 5 untimed calls, then 5 repeats of n back-to-back calls, each bracketed
    # by two events on the launch stream; the median repeat's average call.
    def time_calls(fn, n, repeats=5):
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        per_call = []
        for _ in range(repeats):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for i in range(n):
                fn(i)
            e.record(stream)
            e.synchronize()
            per_call.append(s.elapsed_time(e) / n * 1e3)      # us per call
        return float(np.median(per_call))

    parts = {}
    if do_rswa:
        def rswa_call(i):
            c, rings, out = rswa[i % len(rswa)]
            q, kk, vv = pool[i % 16]
            K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
        us = time_calls(rswa_call, 100)
        nb = algorithmic_bytes_rswa(rs.prefill + rs.window, rs.n_heads)
        parts["rswa_decode_f32"] = {
            "us_per_call": round(us, 2), "algorithmic_bytes": nb,
            "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "kv_positions_per_s": round((rs.prefill + rs.window) / us * 1e6, 1)}

        def rswa_i8_call(i):
            c, rings, out = rswa_i8[i % len(rswa_i8)]
            q, kk, vv = pool[i % 16]
            K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
        us = time_calls(rswa_i8_call, 100)
        nb = algorithmic_bytes_rswa_i8(rs.prefill + rs.window, rs.n_heads)
        parts["rswa_decode_i8"] = {
            "us_per_call": round(us, 2), "algorithmic_bytes": nb,
            "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "kv_positions_per_s": round((rs.prefill + rs.window) / us * 1e6, 1)}

        # [P3] verify_attention on the int8 mirror: 8 drafts, quantised into
        # the workspace, checked against the i8 replicas
        n_draft = 8
        vq_ = t(workloads.normal_f32(workloads.key(rs.seed, 91), (1, n_draft, rs.n_heads, 128)))
        vk_ = t(workloads.normal_f32(workloads.key(rs.seed, 92), (1, n_draft, rs.n_heads, 128)))
        vv_ = t(workloads.normal_f32(workloads.key(rs.seed, 93), (1, n_draft, rs.n_heads, 128)))
        vout = torch.zeros((1, n_draft, rs.n_heads, 128), device=dev)
        vws8 = torch.empty(K.kvq_verify_workspace_bytes(rswa_i8[0][0], rs.n_heads, n_draft), dtype=torch.uint8,
                           device=dev)

        def verify_i8_call(i):
            c, rings, _ = rswa_i8[i % len(rswa_i8)]
            K.rswa_verify(c, rings, rs.n_heads, n_draft, vq_, vk_, vv_, vout, vws8)
        us = time_calls(verify_i8_call, 100)
        rows = rs.prefill + rs.window
        nb = rows * rs.n_heads * 264 + n_draft * rs.n_heads * (512 * 4 + 264 * 2)
        parts["rswa_verify_i8_k8"] = {
            "us_per_call": round(us, 2), "algorithmic_bytes": nb,
            "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "draft_positions_per_s": round(n_draft * rows / us * 1e6, 1)}
        del rswa_i8, vws8

        # prefix-shared reference ([P3] batched_decode_attention's seam): the
        # same 32640-row reference shared by 16 streams, each with its own
        # ring, steady state; 3 replicas (355 MB f32, 92 MB i8 each; the i8
        # replicas do not all exceed the MALL together: 6 of them)
        n_str = 16
        sq = t(workloads.normal_f32(workloads.key(rs.seed, 81), (n_str, rs.n_heads, 128)))
        sk = t(workloads.normal_f32(workloads.key(rs.seed, 82), (n_str, rs.n_heads, 128)))
        sv = t(workloads.normal_f32(workloads.key(rs.seed, 83), (n_str, rs.n_heads, 128)))
        sout = torch.zeros((n_str, rs.n_heads, 128), device=dev)
        rk_d = t(rk.transpose(1, 0, 2))
        rv_d = t(rv.transpose(1, 0, 2))
        for kind, tag, nrep, row_b, app in ((K.KIND_F32, "f32", 3, 1024, K.kv_append_f32),
                                            (K.KIND_I8, "i8", 6, 264, K.kv_append_i8)):
            shared = []
            for rep in range(nrep):
                c = K.KvCache(kind, 1, rs.n_heads, rs.prefill + rs.window * n_str)
                rings = K.Rings(n_str)
                app(c, 0, rs.prefill, rk_d, rv_d)
                K.rswa_shared_record_prefill(c, 0, rings, n_str)
                sws = torch.empty(K.kvq_verify_workspace_bytes(c, rs.n_heads, n_str), dtype=torch.uint8, device=dev)
                for s_ in range(rs.window + 2):
                    K.rswa_shared_decode(c, 0, rings, n_str, rs.n_heads, sq, sk, sv, sout, sws)
                shared.append((c, rings, sws))

            def shared_call(i, shared=shared):
                c, rings, sws = shared[i % len(shared)]
                K.rswa_shared_decode(c, 0, rings, n_str, rs.n_heads, sq, sk, sv, sout, sws)
            us = time_calls(shared_call, 100)
            rows = rs.prefill + rs.window          # visible rows per stream
            # every stored row read once; q read and out written; the step rows
            # read (f32) and written (f32 or codes)
            nb = (rs.prefill + n_str * rs.window) * rs.n_heads * row_b + n_str * rs.n_heads * 512 * 2 \
                + n_str * rs.n_heads * (1024 + 2 * row_b // 2)
            parts["rswa_shared_decode_%s_16_streams" % tag] = {
                "us_per_call": round(us, 2), "algorithmic_bytes": nb,
                "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
                "kv_positions_per_s": round(n_str * rows / us * 1e6, 1)}
            del shared
        del rk_d, rv_d

        # [P3] verify_attention: 8 draft tokens checked against the same
        # replicas, nothing written; bytes as the decode (each row read once
        # for all 8 queries) plus the drafts, queries and outputs
        n_draft = 8
        vq_ = t(workloads.normal_f32(workloads.key(rs.seed, 91), (1, n_draft, rs.n_heads, 128)))
        vk_ = t(workloads.normal_f32(workloads.key(rs.seed, 92), (1, n_draft, rs.n_heads, 128)))
        vv_ = t(workloads.normal_f32(workloads.key(rs.seed, 93), (1, n_draft, rs.n_heads, 128)))
        vout = torch.zeros((1, n_draft, rs.n_heads, 128), device=dev)
        vws = torch.empty(K.kvq_verify_workspace_bytes(rswa[0][0], rs.n_heads, n_draft), dtype=torch.uint8,
                          device=dev)

        def verify_call(i):
            c, rings, _ = rswa[i % len(rswa)]
            K.rswa_verify(c, rings, rs.n_heads, n_draft, vq_, vk_, vv_, vout, vws)
        us = time_calls(verify_call, 100)
        rows = rs.prefill + rs.window
        nb = rows * rs.n_heads * 1024 + n_draft * rs.n_heads * 512 * 4
        flops = 4 * 128 * n_draft * rs.n_heads * (rows + n_draft)
        parts["rswa_verify_f32_k8"] = {
            "us_per_call": round(us, 2), "algorithmic_bytes": nb,
            "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "mfma_TFLOPs": round(flops / us / 1e6, 2),
            "draft_positions_per_s": round(n_draft * rows / us * 1e6, 1)}
    if do_q8:
        def q8_call(i):
            K.decode_attn_q8(cq, bq.n_q_heads, qq, qout, ws_q8)
        us = time_calls(q8_call, 50)
        nb = algorithmic_bytes_q8(cq.len, cq.n_live, bq.n_q_heads)
        parts["decode_attn_q8"] = {
            "us_per_call": round(us, 2), "algorithmic_bytes": nb,
            "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "kv_positions_per_s": round(int(cq.len.sum()) / us * 1e6, 1)}

        # [P3] decode_attention_int8 over the same contexts (per-row int8 K
        # and V, query quantised per head)
        ws_i8 = ci8.workspace(bq.n_q_heads)

        def i8_call(i):
            K.decode_attn_i8(ci8, bq.n_q_heads, qq, qout, ws_i8)
        us = time_calls(i8_call, 50)
        nb = algorithmic_bytes_i8(ci8.len, ci8.n_live, bq.n_q_heads)
        parts["decode_attn_i8"] = {
            "us_per_call": round(us, 2), "algorithmic_bytes": nb,
            "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "kv_positions_per_s": round(int(ci8.len.sum()) / us * 1e6, 1)}
        del ci8, ws_i8

        # [P2] attend_group_upto options: soft-cap 30 and per-Q-head sinks over
        # the full context, then also an 8192-row sliding window
        sinks = t(workloads.normal_f32(workloads.key(bq.seed, 97), (bq.n_q_heads,)) * np.float32(3.0))
        opt_full = K.DecodeOpts(softcap=30.0, sinks=sinks)
        win_first = np.maximum(cq.len.astype(np.int64) - 8192, 0).astype(np.int32)
        opt_win = K.DecodeOpts(first=win_first, softcap=30.0, sinks=sinks)
        for name, o, rows in (("decode_attn_q8_ex_softcap_sinks", opt_full, cq.len),
                              ("decode_attn_q8_ex_window8192_softcap_sinks", opt_win,
                               np.minimum(cq.len, 8192))):
            def ex_call(i, o=o):
                K.decode_attn_q8_ex(cq, bq.n_q_heads, qq, qout, o, ws_q8)
            us = time_calls(ex_call, 50)
            nb = algorithmic_bytes_q8(rows, cq.n_live, bq.n_q_heads)
            parts[name] = {
                "us_per_call": round(us, 2), "algorithmic_bytes": nb,
                "GBps": round(nb / us / 1e3, 1), "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
                "kv_positions_per_s": round(int(np.sum(rows)) / us * 1e6, 1)}

        def app_call(i):
            K.kv_append_q8(cq, K.ALL_SEQS, 1, newk, newv)
        if int(cq.len.max()) + 40 <= cq.capacity:
            parts["kv_append_q8_one_row"] = {"us_per_call": round(time_calls(app_call, 5, repeats=1), 2)}

    if args.part == "small":
        # the three small workloads only: per-call timings, no decode step
        small_parts(parts, K, t, dev, time_calls, log, True, True)
        print(json.dumps({"metric": METRIC, "unit": "KV positions/s", "n_gpus": 1, "parts": parts}), flush=True)
        return

    # ---------------- the timed decode steps ----------------
    # They run after the per-part timing above, so the GPU's clocks have
    # settled when the warm-up steps start (measured: the same step took
    # 485 us after 5 warm-up steps on a cold GPU and 450 us after 100).
    def step(i):
        if do_rswa:
            c, rings, out = rswa[i % len(rswa)]
            q, kk, vv = pool[i % 16]
            K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
        if do_q8:
            K.kv_append_q8(cq, K.ALL_SEQS, 1, newk, newv)
            K.decode_attn_q8(cq, bq.n_q_heads, qq, qout, ws_q8)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # positions attended per step (context rows per sequence)
    pos_rswa = (rs.prefill + rs.window) if do_rswa else 0
    pos_q8 = int(cq.len.sum()) if do_q8 else 0
    positions = pos_rswa + pos_q8
    value = positions / (ms_per_step / 1e3)
    # the step's calls timed on their own (back-to-back calls of each entry
    # point): their sum beside ms_per_step shows what the step adds
    parts_sum_us = round(sum(parts[k]["us_per_call"] for k in ("rswa_decode_f32", "decode_attn_q8",
                                                                 "kv_append_q8_one_row") if k in parts), 2)

    if do_q8:
        # [P1] freeze_cols of one sequence (8 KV heads x 64 rows), the freeze
        # an append of row 64 runs: 64 sequences frozen by 64 back-to-back
        # kv_freeze_col_and_requant calls, bracketed by events.  Bytes per
        # call: each row read once (the requantisation reads it from LDS) and
        # written once, plus the fields.
        fr = K.KvCache(K.KIND_Q8, bq.batch, bq.n_kv_heads, 64)
        fk = t(workloads.normal_f32(workloads.key(bq.seed, 95), (64, bq.n_kv_heads, 128)))
        fv = t(workloads.normal_f32(workloads.key(bq.seed, 94), (64, bq.n_kv_heads, 128)))
        for b in range(bq.batch):
            K.kv_append_q8(fr, b, 64, fk, fv)          # 64 rows: not frozen yet
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s_ev.record(stream)
        for b in range(bq.batch):
            K.kv_freeze_col_and_requant(fr, b)
        e_ev.record(stream)
        e_ev.synchronize()
        us = s_ev.elapsed_time(e_ev) * 1e3 / bq.batch
        nb = bq.n_kv_heads * (64 * 276 * 2 + 2 * 128 * 4)
        parts["kv_freeze_one_seq_64_rows"] = {
            "us_per_call": round(us, 2), "bytes": nb, "GBps": round(nb / us / 1e3, 1)}
        del fr

        # [P2] trim_window over every sequence (window 8192, slack 64, align 64)
        # in one kv_trim_window call: runs once, last, since it shortens the
        # cache.  Bytes: each kept row of each live head read and written once.
        lens_before = cq.len.copy()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s_ev.record(stream)
        _, dropped = K.kv_trim_window(cq, K.ALL_SEQS, [0] * bq.batch, 8192, 64, 64)
        e_ev.record(stream)
        e_ev.synchronize()
        moved = sum(int(lens_before[b]) - int(d) for b, d in enumerate(dropped) if d > 0)
        us = s_ev.elapsed_time(e_ev) * 1e3
        nb = moved * cq.n_live * 276 * 2
        parts["kv_trim_window_all_seqs"] = {
            "us_per_call": round(us, 2), "sequences_trimmed": int(sum(d > 0 for d in dropped)),
            "rows_moved_per_head": moved, "bytes_moved": nb, "GBps": round(nb / us / 1e3, 1),
            "frac_of_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}

    # ---------------- the three small configurations ----------------
    if not args.no_small:
        small_parts(parts, K, t, dev, time_calls, log, do_rswa, do_q8)

    dominant = "decode_attn_q8" if do_q8 else "rswa_decode_f32"
    kernel_tag = "k_decode_q8_batched_q8" if do_q8 else "k_decode_f32_rswa_long_f32"
    d = parts[dominant]
    roofline = {"bound": "hbm", "achieved": d["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac_of_peak"], "traffic": committed_traffic(kernel_tag),
                "kernel": dominant}

    # ---------------- CPU oracle on the host cores ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, rs, bq, do_rswa, do_q8)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "parts_sum_us": parts_sum_us,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32+i8",
        "data": "synthetic (seeded SplitMix64 / Box-Muller; no datasets or weights)",
        "config": {"workload": "decode step: " + " + ".join(
            (["rswa_long_f32 (10 MHA heads x 128, 32640 reference rows + 128-slot ring, f32)"] if do_rswa else [])
            + (["batched_q8 (64 seqs, 32 Q / 8 KV heads x 128, ctx U[1024,32768], q8_2f, +1 appended row/seq)"]
               if do_q8 else [])),
            "positions_per_step": positions, "rswa_replicas": args.replicas if do_rswa else 0},
        "roofline": roofline, "cpu_baseline": cpu, "parts": parts,
    }
    print(json.dumps(rec), flush=True)


def small_parts(parts, K, t, dev, time_calls, log, do_rswa, do_q8):
    """Per-call time of the three small workloads: rswa_f32 (10 heads, 256
    reference rows + full ring), gqa_f32 (32 / 8 heads, 4096 rows, two dead
    groups) and gqa_q8 (32 / 8 heads, 8192 rows).  Each is rotated over
    enough replicas (> 256 MB in all) that the Infinity Cache cannot serve
    repeated reads.  Each is timed as back-to-back calls (us_per_call, which
    includes the host's launch cost at these sizes) and as 200 calls captured
    in one HIP graph and replayed (us_per_call_graph; GB/s and the fraction
    of peak use it).  An R-SWA replay repeats the captured ring write, the
    same work as a step.  These calls are bound by launch and latency more
    than by bandwidth."""
    import torch
    import workloads
    mall = 280e6

    def time_graph(call, n, repeats=5):
        """us per call of n calls captured in one HIP graph and replayed (no
        host launch cost between the calls)."""
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                call(i)
        g.replay()
        torch.cuda.synchronize()
        per_call = []
        for _ in range(repeats):
            s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_ev.record()
            g.replay()
            e_ev.record()
            e_ev.synchronize()
            per_call.append(s_ev.elapsed_time(e_ev) / n * 1e3)
        del g
        return float(np.median(per_call))

    def record(name, call, nb, positions, reps):
        us = time_calls(call, 200)
        try:
            ug = time_graph(call, 200)
        except RuntimeError as e:               # no graph capture here: report the eager timing only
            log("%s: graph timing unavailable (%s)" % (name, e))
            ug = None
        ut = ug if ug is not None else us
        parts[name] = {"us_per_call": round(us, 2), "us_per_call_graph": None if ug is None else round(ug, 2),
                       "algorithmic_bytes": nb, "GBps": round(nb / ut / 1e3, 1),
                       "frac_of_peak": round(nb / ut / 1e3 / HBM_PEAK_GBS, 4),
                       "kv_positions_per_s": round(positions / ut * 1e6, 1), "replicas": reps}

    if do_rswa:
        rs = workloads.get("rswa_f32")
        rows = rs.prefill + rs.window
        nb = algorithmic_bytes_rswa(rows, rs.n_heads)
        reps = int(mall // (rows * rs.n_heads * 1024)) + 1
        rk, rv = rs.reference()
        rk_d, rv_d = t(rk.transpose(1, 0, 2)), t(rv.transpose(1, 0, 2))
        pool = [tuple(t(x[None]) for x in rs.step(s)) for s in range(16)]
        caches = []
        for _ in range(reps):
            c = K.KvCache(K.KIND_F32, 1, rs.n_heads, rows)
            rings = K.Rings(1)
            K.kv_append_f32(c, 0, rs.prefill, rk_d, rv_d)
            K.rswa_record_prefill(c, rings, 0)
            out = torch.zeros((1, rs.n_heads, 128), device=dev)
            for s_ in range(rs.writes - 1):
                q, kk, vv = pool[s_ % 16]
                K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
            caches.append((c, rings, out))
        torch.cuda.synchronize()
        log("rswa_f32 replicas ready: %d" % reps)

        def call(i):
            c, rings, out = caches[i % reps]
            q, kk, vv = pool[i % 16]
            K.rswa_decode(c, rings, rs.n_heads, q, kk, vv, out)
        record("rswa_decode_f32_small", call, nb, rows, reps)
        del caches
    if do_q8:
        for name, kind in (("gqa_f32", K.KIND_F32), ("gqa_q8", K.KIND_Q8)):
            spec = workloads.get(name)
            n = int(spec.lengths()[0])
            alive = spec.alive()
            n_live = int(alive.sum())
            per_row = 1024 if kind == K.KIND_F32 else 276
            nb = (n * n_live * per_row + spec.n_q_heads * 128 * 4 * 2
                  + (n_live * 2 * 128 * 4 if kind == K.KIND_Q8 else 0))
            reps = int(mall // (n * n_live * per_row)) + 1
            k, v = spec.kv_rows(0)
            kd, vd = t(k), t(v)
            app = K.kv_append_f32 if kind == K.KIND_F32 else K.kv_append_q8
            dec = K.decode_attn_f32 if kind == K.KIND_F32 else K.decode_attn_q8
            caches = []
            for _ in range(reps):
                c = K.KvCache(kind, 1, spec.n_kv_heads, n, alive=alive)
                app(c, 0, n, kd, vd)
                caches.append((c, c.workspace(spec.n_q_heads)))
            q = t(spec.query())
            out = torch.zeros((1, spec.n_q_heads, 128), device=dev)
            torch.cuda.synchronize()
            log("%s replicas ready: %d" % (name, reps))

            def call(i, caches=caches, dec=dec, spec=spec, q=q, out=out):
                c, ws = caches[i % len(caches)]
                dec(c, spec.n_q_heads, q, out, ws)
            record("decode_attn_%s_%s" % ("f32" if kind == K.KIND_F32 else "q8", name), call, nb, n, reps)
            del caches


def cpu_baseline(args, rs, bq, do_rswa, do_q8):
    """The oracle as it stands, on the host cores: one decode of the R-SWA
    workload (all 10 heads) and of the first few sequences of the batched q8
    workload (their q8 storage built by the oracle's own codec first, not
    timed).  Reported in the same unit, KV positions/s."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    # The host's core count is reported; the oracle runs one worker per core
    # of this process's CPU share (at most 16: a one-GPU job's share of the
    # host, which a larger pool would oversubscribe).
    host_cores = os.cpu_count() or 1
    try:
        share = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        share = host_cores
    threads = max(1, min(16, share))
    units_r, q_r, units_q, q_q = None, None, None, None
    positions = 0
    if do_rswa:
        rk, rv = rs.reference()
        win_k = np.stack([rs.step(s)[1] for s in range(rs.writes - rs.window, rs.writes)])
        win_v = np.stack([rs.step(s)[2] for s in range(rs.writes - rs.window, rs.writes)])
        q_r = rs.step(rs.writes - 1)[0][None]
        units_r = [[("f32", np.concatenate([rk[g], win_k[:, g]]), np.concatenate([rv[g], win_v[:, g]]))
                    for g in range(rs.n_heads)]]
        positions += rs.prefill + rs.window
    if do_q8:
        nseq = min(args.cpu_sample_seqs, bq.batch)
        lens = bq.lengths()
        q_q = bq.query()[:nseq]
        units_q = []
        for b in range(nseq):
            k, v = bq.kv_rows(b)

            def mk(g):
                h = oracle.Q8Head(cap=int(lens[b]))
                h.append(k[:, g], v[:, g])
                return ("q8", h)
            with ThreadPoolExecutor(threads) as ex:
                units_q.append(list(ex.map(mk, range(bq.n_kv_heads))))
        positions += int(lens[:nseq].sum())
    # the sample decode, repeated until about 10 s of host time has passed
    t0 = time.perf_counter()
    reps = 0
    while True:
        if units_r is not None:
            oracle.decode(q_r, units_r, rs.n_heads, threads=threads)
        if units_q is not None:
            oracle.decode(q_q, units_q, bq.n_kv_heads, threads=threads)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= args.cpu_seconds:
            break
    pos_rep = positions
    positions *= reps
    # one more repeat on a single thread
    t1 = time.perf_counter()
    if units_r is not None:
        oracle.decode(q_r, units_r, rs.n_heads, threads=1)
    if units_q is not None:
        oracle.decode(q_q, units_q, bq.n_kv_heads, threads=1)
    wall1 = time.perf_counter() - t1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    sample = []
    if do_rswa:
        sample.append("rswa_long_f32: one decode, 10 heads x 32768 rows")
    if do_q8:
        sample.append("batched_q8: sequences 0..%d of 64 (%d rows x 8 KV heads x 4 Q heads)"
                      % (args.cpu_sample_seqs - 1, pos_rep - (rs.prefill + rs.window if do_rswa else 0)))
    return {"value": round(positions / wall, 1), "unit": "KV positions/s", "cores": threads,
            "host_cores": host_cores, "cpu_affinity": share,
            "kind": "oracle", "sample": "; ".join(sample) + "; float64 oracle, repeated %d times, %.2f s wall"
            % (reps, wall),
            "single_core_value": round(pos_rep / wall1, 1), "cpu_model": model}


if __name__ == "__main__":
    main()
