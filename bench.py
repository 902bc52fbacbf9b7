#!/usr/bin/env python3
"""Benchmark of the HeadPrep + attention path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs:
  1. HeadPrep of k in place (attn_prep)                       -- bf16 prefill workload
  2. causal attention with q's HeadPrep fused (attn_prefill)   -- bf16 prefill workload
  3. single-row decode against a 4096-row KV cache (attn_decode) -- bf16 decode workload
Workloads: prefill batch 4 x 2048 tokens, 32 q heads over 8 kv heads, d 128 (rotary
base 1e4); decode batch 32, 32 q heads over 8 kv heads, d 128, cache 4096 rows, query
at position 4096.  Inputs are seeded synthetic N(0, 1) operands (synthetic.py) already
resident in HBM; the decode step rotates through several cache copies so repeats are
not served from the 256 MB last-level cache.

After the timed steps: the long prefill workload (batch 1 x 16384 tokens, 64 q / 8 kv
heads, rotary base 1e6, 1 % outlier key rows), k HeadPrep + attention per call; the
chunked prefill workload (batch 4: 512 new tokens appended to a 3584-row cache, 32 q / 8
kv heads, attention over all 4096 rows) per attn_prefill_chunk call; the decode workload
against caches coded in 8/8, 4/4 and 4/2 bits (attn_decode_q; GB/s of the codes, their
ranges, q and out); packed rows of an
image model (attn_rows: 4608 rows of 24 heads of 128, HeadPrep with adjacent pairs in
place -- repeated calls re-prep the same buffer, which changes values, not work -- then
full attention), and the same rows through the quantised path (attn_rows8: 8-bit coding
pass + Q K^T on INT8, P V on E4M3); the whole-row norm + per-head rotary of 6240 rows of 4096
(attn_row_norm_rope, in place, GB/s of one read and one write plus the tables); then two
calibration kernels (libpeak.so: a bf16 MFMA loop and a streaming read) give measured
ceilings next to the published ones.

Printed: one JSON line.  `value` is the prefill rate (algorithmic flops of the visible
causal pairs, 4 d per (query, key, head), over the mean time of steps 1-2); the decode
rate (algorithmic bytes over the mean time of step 3) is under "decode".  `roofline` is
the attention kernel's (step 2 alone), `decode_roofline` the decode call's, both timed
with HIP events on the launch stream.  `traffic` is the HBM bytes per launch read from
profiles/traffic.json (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a plain copy), or
null when the kernel sources changed since those counters were taken.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E (published)
PEAK_8BIT_TFLOPS = 5000.0      # MI355X dense int8 / fp8 MFMA (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def prefill_flops(w) -> int:
    pairs = w.seq * (w.seq + 1) // 2 if w.causal else w.seq * w.seq
    return 4 * w.d * pairs * w.batch * w.hq


def decode_bytes(w) -> int:
    kv = 2 * w.batch * w.seq * w.hkv * w.d * 2
    qo = 2 * w.batch * w.hq * w.d * 2
    return kv + qo + 2 * w.half * 4 + w.d * 4     # + one cos/sin table row + qw


def sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per launch from the committed counter run, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if sources_sha(rec["sources"]) != rec["sources_sha256"]:
        return None
    return rec["bytes_per_launch"]


def host_cpu_model() -> str:
    """The host CPU's model name as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, inp) -> dict:
    """The f64 oracle, as it stands, on the full prefill workload (HeadPrep of q and k
    plus attention of every query row) on this host's cores."""
    import oracle
    t0 = time.perf_counter()
    oracle.prefill(inp["q"], inp["k"], inp["v"], inp["qw"], inp["kw"], inp["cos"], inp["sin"],
                   w.half, w.eps, 0, w.scale, True)
    dt = time.perf_counter() - t0
    return {"value": round(prefill_flops(w) / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": "the whole bf16 prefill workload (4 x 2048 tokens, 32/8 heads, d 128): "
                      "HeadPrep of q and k and causal attention of every row, f64, %.1f s" % dt,
            "host_cpu": host_cpu_model(), "cores_in_affinity_mask": len(os.sched_getaffinity(0))}


def decode_bytes_q(w, kbits: int, vbits: int) -> int:
    """Bytes a quantised-cache decode must move: the codes of every cached key and value
    of every kv head, their (lo, step) pairs, q and out (bf16), one table row and qw."""
    rows = w.batch * w.seq * w.hkv
    return (rows * w.d * (kbits + vbits) // 8 + rows * 2 * 8 + 2 * w.batch * w.hq * w.d * 2 +
            (2 * w.half + w.d) * 4)


def stats_ms(a) -> dict:
    import numpy as np
    a = np.asarray(a)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "min": round(float(a.min()), 5)}


def measured_peaks(torch, dev) -> dict:
    """Best of a few runs of the two calibration kernels."""
    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_headprep_amd", "libpeak.so"))
    lib.peak_mfma_bf16_flops.restype = ctypes.c_double
    lib.peak_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)

    def best(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        return min(times)

    blocks, iters = 512, 4000                  # 2 waves per SIMD on 256 CUs
    t = best(lambda: lib.peak_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()), sp))
    mfma = lib.peak_mfma_bf16_flops(blocks, iters) / t / 1e12
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    t = best(lambda: lib.peak_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), sp))
    del buf
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_gbps": round(nbytes / t / 1e9, 1),
            "how": "libpeak.so: %d blocks x 4 waves x %d rounds of 8 independent "
                   "v_mfma_f32_32x32x16_bf16; a grid-stride 16-byte read of 1 GiB; best of 5" % (blocks, iters)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cache-copies", type=int, default=3)
    ap.add_argument("--long-calls", type=int, default=20, help="timed calls of the long prefill (0: skip)")
    ap.add_argument("--paged-calls", type=int, default=30, help="timed calls of the paged decode (0: skip)")
    ap.add_argument("--chunk-calls", type=int, default=20, help="timed calls of the chunked prefill (0: skip)")
    ap.add_argument("--quant-calls", type=int, default=30,
                    help="timed calls of the decode against 8/8, 4/4 and 4/2-bit caches (0: skip)")
    ap.add_argument("--rows-calls", type=int, default=20,
                    help="timed calls of the packed-rows attention and the row norm (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the calibration kernels")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), to scale HBM "
                         "byte counters read by a profiler")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path is built and timed on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synthetic
    import transformer_attention_headprep_amd as tah

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n, "copies": 5}))
        return 0

    def to(x, dt="bf16"):
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return (t.to(torch.bfloat16) if dt == "bf16" else t).to(dev)

    wp = synthetic.WORKLOADS["prefill_bf16"]
    wd = synthetic.WORKLOADS["decode_bf16"]
    ip = synthetic.make_prefill(wp)
    idc = synthetic.make_decode(wd)

    # prefill operands
    q3, k3, v3 = to(ip["q"]), to(ip["k"]), to(ip["v"])
    out3 = torch.empty_like(q3)
    prep3 = tah.HeadPrep(to(ip["qw"], "f32"), to(ip["kw"], "f32"), to(ip["cos"], "f32"),
                         to(ip["sin"], "f32"), wp.eps)
    # k already prepped (by attn_prep with kw): its rows' norms are within key_bound(kw)
    prep3_q = tah.HeadPrep(prep3.qw, None, prep3.cos, prep3.sin, wp.eps, kmax=tah.key_bound(ip["kw"], wp.d))

    # decode operands: caches prepped on the GPU (HeadPrep at positions 0 .. 4095)
    prep4 = tah.HeadPrep(to(idc["qw"], "f32"), to(idc["kw"], "f32"), to(idc["cos"], "f32"),
                         to(idc["sin"], "f32"), wd.eps)
    q4 = to(idc["q"])
    k_raw = to(idc["k_raw"])
    tah.attn_prep(None, k_raw, prep4, pos0=0)
    kcs = [k_raw] + [k_raw.clone() for _ in range(args.cache_copies - 1)]
    v_raw = to(idc["v"])
    vcs = [v_raw] + [v_raw.clone() for _ in range(args.cache_copies - 1)]
    lens = torch.tensor(idc["lens"], device=dev)
    pos = torch.tensor(idc["pos"], device=dev)
    splits = tah.decode_default_splits(wd.batch, wd.hq, wd.hkv, wd.d, wd.seq)
    need = tah.decode_workspace_size(wd.batch, wd.hq, wd.hkv, wd.d, wd.seq, splits)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    out4 = torch.empty_like(q4)
    stream = torch.cuda.current_stream()

    def time_calls(fn, calls):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        torch.cuda.synchronize()
        # The calls are queued behind a spin kernel (about 150 us a call), so each pair of
        # events times one call's GPU work, not the host marshalling of its arguments
        # (which can take longer than a short call runs).
        torch.cuda._sleep(int(calls * 150e-6 * 2.1e9))
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        tah.attn_prep(None, k3, prep3, pos0=0, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        tah.attn_prefill(q3, k3, v3, out3, prep=prep3_q, causal=True, scale=wp.scale, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        c = i % len(kcs)
        tah.attn_decode(q4, kcs[c], vcs[c], lens, pos, wd.seq, prep=prep4, scale=wd.scale,
                        splits=splits, workspace=ws, out=out4, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    prep_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    attn_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in events])
    flops = prefill_flops(wp)
    nbytes = decode_bytes(wd)
    pre_tflops = flops / ((prep_ms + attn_ms).mean() * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms.mean() * 1e-3) / 1e12
    dec_gbps = nbytes / (dec_ms.mean() * 1e-3) / 1e9
    # ---- decode against quantised caches (coded on the GPU from the same prepped caches)
    quant_lines = {}
    if args.quant_calls > 0:
        for kb, vb in ((8, 8), (4, 4), (4, 2)):
            qk, qv = [], []
            for c in range(len(kcs)):
                kq = tah.QuantCache.empty(wd.batch, wd.hkv, wd.seq, wd.d, kb, device=dev)
                vq = tah.QuantCache.empty(wd.batch, wd.hkv, wd.seq, wd.d, vb, device=dev)
                tah.attn_kv_quantize(kcs[c], kq, row0=0)
                tah.attn_kv_quantize(vcs[c], vq, row0=0)
                qk.append(kq)
                qv.append(vq)
            turn = [0]
            sq = tah.decode_q_default_splits(wd.batch, wd.hq, wd.hkv, wd.seq, kb)
            nq = tah.decode_workspace_size(wd.batch, wd.hq, wd.hkv, wd.d, wd.seq, sq)
            wsq = torch.empty(nq, dtype=torch.uint8, device=dev) if nq else None

            def callq():
                c = turn[0] % len(qk)
                turn[0] += 1
                tah.attn_decode_q(q4, qk[c], qv[c], lens, pos, wd.seq, prep=prep4, scale=wd.scale, splits=sq,
                                  workspace=wsq, out=out4, stream=stream)

            msq = time_calls(callq, args.quant_calls)
            qbytes = decode_bytes_q(wd, kb, vb)
            gbq = qbytes / (msq.mean() * 1e-3) / 1e9
            quant_lines["k%d_v%d" % (kb, vb)] = {
                "value": round(gbq, 2), "unit": "GB/s", "ms": stats_ms(msq), "bytes": qbytes,
                "frac_of_hbm_peak": round(gbq / PEAK_HBM_GBPS, 4), "splits": sq,
                "speedup_vs_bf16_cache": round(float(dec_ms.mean() / msq.mean()), 3)}
            del qk, qv
        torch.cuda.empty_cache()

    # ---- the same decode through a paged pool: 64-row pages in a random order
    paged_line = None
    if args.paged_calls > 0:
        page_rows = 64
        per_seq = wd.seq // page_rows
        num_pages = wd.batch * per_seq
        perm = torch.from_numpy(np.random.default_rng(7).permutation(num_pages).astype(np.int64)).to(dev)
        table = perm.view(wd.batch, per_seq).to(torch.int32).contiguous()
        kps, vps = [], []
        for c in range(len(kcs)):
            kp = torch.empty_like(kcs[c]).view(num_pages, page_rows, wd.hkv, wd.d)
            vp = torch.empty_like(vcs[c]).view(num_pages, page_rows, wd.hkv, wd.d)
            kp[perm] = kcs[c].view(num_pages, page_rows, wd.hkv, wd.d)
            vp[perm] = vcs[c].view(num_pages, page_rows, wd.hkv, wd.d)
            kps.append(kp)
            vps.append(vp)
        turn = [0]

        def callp():
            c = turn[0] % len(kps)
            turn[0] += 1
            tah.attn_decode_paged(q4, kps[c], vps[c], table, lens, pos, wd.seq, prep=prep4, scale=wd.scale,
                                  splits=splits, workspace=ws, out=out4, stream=stream)

        msp = time_calls(callp, args.paged_calls)
        gbp = nbytes / (msp.mean() * 1e-3) / 1e9
        paged_line = {"workload": "the bf16 decode workload read through a paged pool (64-row pages, the page "
                                  "table a random permutation), 3 pools in turn",
                      "value": round(gbp, 2), "unit": "GB/s", "ms": stats_ms(msp), "bytes": nbytes,
                      "frac_of_hbm_peak": round(gbp / PEAK_HBM_GBPS, 4),
                      "vs_contiguous": round(float(dec_ms.mean() / msp.mean()), 3)}
        del kps, vps
        torch.cuda.empty_cache()

    del q3, k3, v3, out3, kcs, vcs, k_raw, v_raw

    # ---- long prefill: k HeadPrep + attention per call
    long_line = None
    if args.long_calls > 0:
        wl = synthetic.WORKLOADS["long_prefill_bf16"]
        il = synthetic.make_prefill(wl)
        q5, k5, v5 = to(il["q"]), to(il["k"]), to(il["v"])
        out5 = torch.empty_like(q5)
        prep5 = tah.HeadPrep(to(il["qw"], "f32"), to(il["kw"], "f32"), to(il["cos"], "f32"),
                             to(il["sin"], "f32"), wl.eps)
        prep5_q = tah.HeadPrep(prep5.qw, None, prep5.cos, prep5.sin, wl.eps, kmax=tah.key_bound(il["kw"], wl.d))

        def call5():
            tah.attn_prep(None, k5, prep5, pos0=0, stream=stream)
            tah.attn_prefill(q5, k5, v5, out5, prep=prep5_q, causal=True, scale=wl.scale, stream=stream)

        for _ in range(3):
            call5()
        ev5 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.long_calls)]
        torch.cuda.synchronize()
        for a, b in ev5:
            a.record(stream)
            call5()
            b.record(stream)
        torch.cuda.synchronize()
        ms5 = np.array([a.elapsed_time(b) for a, b in ev5])
        tf5 = prefill_flops(wl) / (ms5.mean() * 1e-3) / 1e12
        long_line = {"workload": "bf16 long prefill (batch 1, seq 16384, 64 q / 8 kv heads, d 128, "
                                 "rotary base 1e6, 1 % outlier key rows), k HeadPrep + attention",
                     "value": round(tf5, 3), "unit": "TFLOP/s", "calls": args.long_calls,
                     "ms": stats_ms(ms5), "flops": prefill_flops(wl),
                     "frac_of_bf16_peak": round(tf5 / PEAK_BF16_TFLOPS, 4)}
        del q5, k5, v5, out5
        torch.cuda.empty_cache()

    # ---- chunked prefill: append 512 tokens to a 3584-row cache and attend all 4096
    chunk_line = None
    if args.chunk_calls > 0:
        wc = synthetic.WORKLOADS["chunk_prefill_bf16"]
        n_past, tq = wc.extra["n_past"], wc.extra["tq"]
        ic = synthetic.make_prefill(wc)
        prep6 = tah.HeadPrep(to(ic["qw"], "f32"), to(ic["kw"], "f32"), to(ic["cos"], "f32"),
                             to(ic["sin"], "f32"), wc.eps, kmax=tah.key_bound(ic["kw"], wc.d))
        kc6, vc6 = to(ic["k"]), to(ic["v"])                  # [4, 4096, 8, 128]: the cache
        tah.attn_prep(None, kc6, prep6, pos0=0)              # rows 0 .. 3583 hold prepped keys
        q6 = to(ic["q"][:, n_past:])
        kn6, vn6 = to(ic["k"][:, n_past:]), to(ic["v"][:, n_past:])
        out6 = torch.empty_like(q6)

        def call6():
            tah.attn_prefill_chunk(q6, kn6, vn6, kc6, vc6, n_past, out=out6, prep=prep6, causal=True,
                                   scale=wc.scale, stream=stream)

        for _ in range(3):
            call6()
        ev6 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.chunk_calls)]
        torch.cuda.synchronize()
        for a, b in ev6:
            a.record(stream)
            call6()
            b.record(stream)
        torch.cuda.synchronize()
        ms6 = np.array([a.elapsed_time(b) for a, b in ev6])
        pairs6 = sum(n_past + i + 1 for i in range(tq))
        flops6 = 4 * wc.d * pairs6 * wc.batch * wc.hq
        tf6 = flops6 / (ms6.mean() * 1e-3) / 1e12
        chunk_line = {"workload": "bf16 chunked prefill (batch 4, 512 new tokens after 3584 cached, 32 q / 8 kv "
                                  "heads, d 128): k HeadPrep + cache append + attention over 4096 rows",
                      "value": round(tf6, 3), "unit": "TFLOP/s", "calls": args.chunk_calls,
                      "ms": stats_ms(ms6), "flops": flops6,
                      "frac_of_bf16_peak": round(tf6 / PEAK_BF16_TFLOPS, 4)}
        del q6, kn6, vn6, out6, kc6, vc6
        torch.cuda.empty_cache()

    # ---- packed image-model rows: HeadPrep (adjacent pairs) in place + full attention
    rows_line = None
    if args.rows_calls > 0:
        n7, heads7, head7 = 4608, 24, 128
        rng7 = np.random.default_rng(7)
        qkv7 = to(synthetic.bf16_round(rng7.standard_normal((n7, 3 * heads7 * head7))))
        cos7, sin7 = synthetic.rope_tables(n7, head7 // 2, head7, 1e4)
        prep7 = tah.HeadPrep(to(rng7.uniform(0.5, 1.5, head7), "f32"), to(rng7.uniform(0.5, 1.5, head7), "f32"),
                             to(cos7, "f32"), to(sin7, "f32"), 1e-6, pairs=True)
        out7 = torch.empty(n7, heads7 * head7, dtype=torch.bfloat16, device=dev)
        ms7 = time_calls(lambda: tah.attn_rows(qkv7, heads7, head7, out=out7, prep=prep7, stream=stream),
                         args.rows_calls)
        flops7 = 4 * head7 * n7 * n7 * heads7
        tf7 = flops7 / (ms7.mean() * 1e-3) / 1e12
        rows_line = {"workload": "bf16 packed rows of an image model (4608 rows = 4096 image + 512 text, 24 heads "
                                 "of 128, full attention, HeadPrep with adjacent pairs in place)",
                     "value": round(tf7, 3), "unit": "TFLOP/s", "calls": args.rows_calls,
                     "ms": stats_ms(ms7), "flops": flops7, "frac_of_bf16_peak": round(tf7 / PEAK_BF16_TFLOPS, 4)}
        # the same rows through the quantised path: HeadPrep + 8-bit coding pass, then
        # Q K^T on INT8 and P V on E4M3 (qkv is not written)
        total8, _ = tah.rows8_layout(n7, heads7, head7)
        ws8 = torch.empty(total8, dtype=torch.uint8, device=dev)
        ms8a = time_calls(lambda: tah.attn_rows8(qkv7, heads7, head7, out=out7, prep=prep7, workspace=ws8,
                                                 stream=stream), args.rows_calls)
        ms8b = time_calls(lambda: tah.attn_rows8_attend(ws8, n7, heads7, head7, out=out7, stream=stream),
                          args.rows_calls)
        tf8a = flops7 / (ms8a.mean() * 1e-3) / 1e12
        tf8b = flops7 / (ms8b.mean() * 1e-3) / 1e12
        rows_line["quantized"] = {
            "value": round(tf8a, 3), "unit": "TFLOP/s", "ms": stats_ms(ms8a),
            "attention_only": {"value": round(tf8b, 3), "ms": stats_ms(ms8b),
                               "frac_of_int8_fp8_peak": round(tf8b / PEAK_8BIT_TFLOPS, 4)},
            "speedup_vs_bf16": round(float(ms7.mean() / ms8a.mean()), 3)}
        del ws8
        del qkv7, out7
        torch.cuda.empty_cache()

    # ---- whole-row norm + per-head rotary of a video model's q (HBM-bound, in place)
    rownorm_line = None
    if args.rows_calls > 0:
        r8, w8, h8 = 6240, 4096, 128
        rng8 = np.random.default_rng(8)
        ang8 = rng8.uniform(-np.pi, np.pi, (r8, w8 // 2))
        wt8 = to(rng8.uniform(0.5, 1.5, w8), "f32")
        # three copies of rows and tables in turn (613 MB), so no call finds its operands in the
        # 256 MB last-level cache
        x8s = [to(synthetic.bf16_round(rng8.standard_normal((r8, w8)))) for _ in range(3)]
        cos8s = [to(np.cos(ang8), "f32") for _ in range(3)]
        sin8s = [to(np.sin(ang8), "f32") for _ in range(3)]
        turn8 = [0]

        def call8():
            i = turn8[0] % 3
            turn8[0] += 1
            tah.attn_row_norm_rope(x8s[i], wt8, 1e-6, cos8s[i], sin8s[i], head=h8, stream=stream)

        ms8 = time_calls(call8, args.rows_calls)
        bytes8 = r8 * w8 * 2 * 2 + r8 * (w8 // 2) * 4 * 2 + w8 * 4
        gb8 = bytes8 / (ms8.mean() * 1e-3) / 1e9
        rownorm_line = {"workload": "bf16 whole-row norm + per-head rotary in place (6240 rows of 4096 = 32 heads "
                                    "of 128: an 832 x 480, 124-frame video's latent rows)",
                        "value": round(gb8, 2), "unit": "GB/s", "calls": args.rows_calls, "ms": stats_ms(ms8),
                        "bytes": bytes8, "frac_of_hbm_peak": round(gb8 / PEAK_HBM_GBPS, 4)}
        del x8s, cos8s, sin8s
        torch.cuda.empty_cache()

    peaks = None if args.no_peaks else measured_peaks(torch, dev)

    line = {
        "metric": "prefill attention TFLOP/s + decode HBM GB/s (HeadPrep fused), 1 MI355X",
        "value": round(pre_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) operands, U(0.5,1.5) norm weights, f32 rotary tables)",
        "config": {
            "workload": "bf16 prefill (batch 4, seq 2048, 32 q / 8 kv heads, d 128, causal) + "
                        "bf16 decode (batch 32, cache 4096, 32 q / 8 kv heads, d 128)",
            "prefill": {"batch": wp.batch, "seq": wp.seq, "hq": wp.hq, "hkv": wp.hkv, "d": wp.d,
                        "half": wp.half, "rotary_base": wp.base, "causal": True},
            "decode": {"batch": wd.batch, "cache": wd.seq, "query_position": wd.seq, "hq": wd.hq,
                       "hkv": wd.hkv, "d": wd.d, "splits": splits, "cache_copies": args.cache_copies},
        },
        "parts_ms": {"k_headprep": stats_ms(prep_ms), "prefill_attention": stats_ms(attn_ms),
                     "decode": stats_ms(dec_ms)},
        "decode": {"value": round(dec_gbps, 2), "unit": "GB/s", "bytes": nbytes,
                   "frac_of_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4)},
        "roofline": {"kernel": "prefill_bf16_kernel (attention, q HeadPrep fused)",
                     "bound": "mfma", "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_bf16_kernel"), "flops_per_launch": flops},
        "decode_roofline": {"kernel": "decode_rows_kernel + decode_merge_kernel (q HeadPrep fused, %d key splits)" % splits,
                            "bound": "hbm", "achieved": round(dec_gbps, 2), "peak": PEAK_HBM_GBPS,
                            "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                            "traffic": recorded_traffic("decode_rows_kernel"), "bytes_per_launch": nbytes},
    }
    if long_line is not None:
        line["long_prefill"] = long_line
    if chunk_line is not None:
        line["chunk_prefill"] = chunk_line
    if paged_line is not None:
        line["decode_paged"] = paged_line
    if quant_lines:
        line["decode_quantized"] = dict(
            workload="bf16 decode workload against quantised caches (keys and values in k / v bits, per-head "
                     "least-squared-error ranges), 3 cache copies in turn", **quant_lines)
    if rows_line is not None:
        line["image_rows"] = rows_line
    if rownorm_line is not None:
        line["row_norm_rope"] = rownorm_line
    if peaks is not None:
        peaks["prefill_attention_frac"] = round(attn_tflops / peaks["mfma_bf16_tflops"], 4)
        peaks["decode_frac"] = round(dec_gbps / peaks["hbm_read_gbps"], 4)
        line["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wp, ip)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
