#!/usr/bin/env python3
"""Benchmark of the coalesced attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one coalesced forward launch over the mixed rank share: one
theta = (4, 1, 1) shard of a 32760-token video (8190 queries against all
32760 keys) packed with 24 whole 1024-token and 32 whole 256-token images,
24 heads, head_dim 128, bf16 inputs already resident in HBM. The worklist is
built once per batch on the host (timed separately) and reused, as every
layer of a training step reuses it. Prints one JSON line.

The other steps of the path are timed beside it in the same run: the
KV-split merge (two 27450-row partials on 12 heads, reported in GB/s) and
the recompute-from-LSE backward of the same mix with an upstream gradient
(reported in TFLOP/s under both flop conventions: 5 GEMMs = 2.5x the
forward's flops, and 4 GEMMs = 2x). The ``configs`` object times the
forward on the other workloads (the tiny check, images only, the KV-split
shard with its merge, with and without the in-launch key split, and the two
second-workload shares), and ``price_table`` gives the additivity ratios of
the mixed rank share. Every GPU time comes from HIP events on the launch
stream; medians and minima are reported beside the means. ``mfma_attainable``
gives the rate of a register-only bf16 MFMA stream on this GPU, on random and
on constant operands: the chip is power-limited, and the random figure is the
matrix-core rate it attains on data like the workload's. The cpu_baseline
leg times the fp64 oracle on a bounded sample of the same workload on the
host cores (one thread per core, single-threaded BLAS).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "mixed-batch coalesced attention fwd TFLOP/s and % of bf16 MFMA peak"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload index (2 = mixed rank share)")
    ap.add_argument("--n-slots", type=int, default=-1, help="static slots (-1: one per CU, 0: one WG per tile)")
    ap.add_argument("--kv-chunk", type=int, default=0,
                    help="split items with more keys into key chunks merged inside the forward (0: off)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config forward records (configs 0, 1, 3, 5, 6)")
    ap.add_argument("--no-price", action="store_true", help="skip the additivity ratios")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time")
    ap.add_argument("--price-table", action="store_true",
                    help="instead of the bench line: per-(bucket, theta) prices of the workload's items "
                         "alone and per bucket, against the coalesced launch (additivity check)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (scale reference for FETCH/WRITE_SIZE)")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="only time the register-only bf16 MFMA stream on random and constant operands")
    ap.add_argument("--no-calib", action="store_true",
                    help="leave the MFMA calibration out of the bench line")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(files):
    """sha256 over the sources a profiled kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads for a
    plain copy of known size), or None when the record is missing or the
    kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC) as fh:
            rec = json.load(fh)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash(rec["sources"]):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def _events_ms(fn, steps, stream):
    """Average duration of fn() over `steps` launches, from HIP events
    recorded on the stream the kernels run on."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / steps


def _launch_ms(fn, steps, stream):
    """Duration of each of `steps` calls of fn(), from a pair of HIP events
    around each call on the stream the kernels run on."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
    evs[-1][1].synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def _spread(ms):
    ms = sorted(ms)
    return {"ms_mean": round(sum(ms) / len(ms), 4), "ms_median": round(float(np.median(ms)), 4),
            "ms_min": round(ms[0], 4), "ms_max": round(ms[-1], 4), "launches": len(ms)}


def _cpu_baseline(wl, inp, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    one worker thread per host core (at most 16, the share of the host one
    GPU gets), each running (item, head) units with single-threaded BLAS
    (numpy releases the interpreter lock inside its array kernels)."""
    import threading
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle.attention import coalesced_forward_rows
    from coalesced_attention_amd.workloads import sample_rows
    host_cpus = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host_cpus))
    Qh, Kh, Vh = (x.float().numpy() for x in (inp.q, inp.k, inp.v))
    s = wl.softmax_scale
    d = wl.head_dim

    # pass 0: the rows the parity tests check (every row of short items,
    # four per 128-row block of long ones), in a seeded random order of
    # (item, head) units; later passes: fresh seeded rows of the long items;
    # stop once the target time is spent
    def units():
        pass_no = 0
        while True:
            out = []
            for idx, it in enumerate(wl.items):
                if pass_no > 0 and it.q_len <= 1024:
                    continue
                rows = sample_rows(it, seed=idx + 1000 * pass_no)
                for h in range(it.head_begin, it.head_begin + it.head_cnt):
                    out.append((pass_no, it, h, rows))
            for i in np.random.default_rng(pass_no).permutation(len(out)):
                yield out[i]
            pass_no += 1

    gen = units()
    lock = threading.Lock()
    t0 = time.perf_counter()

    def worker():
        flops = rows_done = last_pass = 0
        while True:
            with lock:
                if time.perf_counter() - t0 > target_s:
                    break
                pass_no, it, h, rows = next(gen)
            coalesced_forward_rows(Qh, Kh, Vh, it, h, rows, s)
            flops += 4 * len(rows) * it.kv_len * d
            rows_done += len(rows)
            last_pass = max(last_pass, pass_no)
        return flops, rows_done, last_pass

    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        res = [f.result() for f in [ex.submit(worker) for _ in range(workers)]]
    el = time.perf_counter() - t0
    flops = sum(r[0] for r in res)
    rows_done = sum(r[1] for r in res)
    passes = max(r[2] for r in res) + 1
    total_rows = sum(it.q_len * it.head_cnt for it in wl.items)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "host_cpus": host_cpus, "blas_threads_per_worker": 1,
            "sample": f"{rows_done} (query row, head) pairs of the same workload ({total_rows} in all): "
                      f"every image row and 4 rows per 128-row block of the video shard, then "
                      f"fresh rows of the shard ({passes} pass(es); {flops / 1e9:.1f} GFLOP in "
                      f"{el:.1f} s, fp64 numpy, {workers} worker threads)"}


def _bench_backward(zl, W, dev, stream, n_slots):
    """Backward of the training-step mix (the mixed rank share plus dO):
    forward once for O and LSE, then timed backward launches (D preprocess
    and the key-block kernel) accumulating into zeroed fp32 gradients."""
    import torch
    wl = W.config(4)
    inp = W.make_inputs(wl)
    q, k, v, g = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dout))
    del inp
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim,
                              n_slots=n_slots)
    built.to(dev)
    o, lse = zl.coalesced_attn_fwd(built, q, k, v, stream=stream)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(lse.shape, dtype=torch.float32, device=dev)

    def bwd():
        zl.coalesced_attn_bwd(built, q, k, v, o, lse, g, dq, dk, dv, ws, stream=stream)

    def zero():
        dq.zero_()
        dk.zero_()
        dv.zero_()

    for _ in range(2):
        bwd()
    torch.cuda.synchronize()
    sp = _spread(_launch_ms(bwd, 10, stream))
    ms = sp["ms_mean"]
    zms = _events_ms(zero, 10, stream)
    F = wl.flops_fwd()
    return {"workload": wl.name, "ms": round(ms, 4), "ms_median": sp["ms_median"], "ms_min": sp["ms_min"],
            "zero_grads_ms": round(zms, 4),
            "TFLOP/s": round(2.5 * F / (ms * 1e-3) / 1e12, 2),
            "TFLOP/s_4gemm": round(2.0 * F / (ms * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100 * 2.5 * F / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "flops_5gemm": 2.5 * F, "bwd_tiles": built.header.n_bwd_tiles}


def _price_table(zl, wl, q, k, v, dev, n_slots):
    """Per-(bucket, theta) prices on this GPU. A bucket is one item shape
    (q_len, kv_len, head_cnt); the theta split of a shard shows in that shape.
    For each bucket: one item alone, and all of the bucket's items in one
    launch; then the whole mix coalesced. The pages' planner prices a batch
    as the sum of per-item prices; coalesced / sum says how additive this
    kernel is."""
    import torch
    from collections import OrderedDict
    stream = torch.cuda.current_stream(dev)
    o = torch.empty((wl.q_rows, wl.num_heads, wl.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.q_rows, wl.num_heads), dtype=torch.float32, device=dev)

    def timed(items):
        built = zl.build_worklist(items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim,
                                  n_slots=n_slots, device=dev)
        run = lambda: zl.coalesced_attn_fwd(built, q, k, v, o, lse, stream=stream)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        ms = _events_ms(run, 3, stream)
        reps = max(3, min(200, int(60.0 / max(ms, 1e-3))))  # ~60 ms of launches
        return _events_ms(run, reps, stream)

    buckets = OrderedDict()
    for it in wl.items:
        buckets.setdefault((it.q_len, it.kv_len, it.head_cnt), []).append(it)
    rows = []
    for (ql, kl, hc), its in buckets.items():
        single = timed(its[:1])
        whole = timed(its)
        rows.append({"q_len": ql, "kv_len": kl, "head_cnt": hc, "count": len(its),
                     "single_ms": round(single, 4), "bucket_ms": round(whole, 4),
                     "flops": 4 * ql * kl * hc * wl.head_dim * len(its)})
    coalesced = timed(wl.items)
    sum_single = sum(r["single_ms"] * r["count"] for r in rows)
    sum_bucket = sum(r["bucket_ms"] for r in rows)
    return {"metric": "coalesced launch time / sum of isolated prices", "workload": wl.name,
            "n_slots": n_slots, "buckets": rows, "coalesced_ms": round(coalesced, 4),
            "sum_single_prices_ms": round(sum_single, 4), "sum_bucket_launches_ms": round(sum_bucket, 4),
            "coalesced_over_single_prices": round(coalesced / sum_single, 4),
            "coalesced_over_bucket_launches": round(coalesced / sum_bucket, 4),
            "data": "synthetic"}


def _calibrate_mfma(zl, iters=400_000):
    """Rate of a register-only stream of bf16 32x32x16 MFMAs on this GPU
    (``zl_calib_mfma``), on random and on constant operands: under its power
    limit the chip attains less than the nominal peak when the operand bits
    switch, and the random figure is the ceiling a kernel on random data
    meets on this GPU."""
    return {"random_bf16": round(zl.calibrate_mfma("random", iters), 1),
            "constant_bf16": round(zl.calibrate_mfma("constant", iters), 1),
            "unit": "TFLOP/s", "iters": iters, "kernel": "mfma_stream"}


def _bench_configs(zl, W, dev, stream, n_slots):
    """Forward time of the other workloads: the tiny check (microseconds),
    images only, the KV-split shard with its theta-k merge (with and without
    the in-launch key split), and the two second-workload shares (with and
    without the automatic key split, which cuts their long items into
    chunks of at most 65,536 keys merged inside the launch). HIP events
    around each launch; ~20 launches after 3 warm-ups (fewer on the long
    ones)."""
    import torch
    out = {}
    for c, kv_chunk in ((0, 0), (1, 0), (3, 0), (3, 27456), (3, 65536), (5, 0), (5, zl.KV_CHUNK_AUTO),
                        (6, 0), (6, zl.KV_CHUNK_AUTO)):
        wl = W.config(c)
        inp = W.make_inputs(wl)
        q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
        del inp
        built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim,
                                  n_slots=n_slots, kv_chunk=kv_chunk)
        built.to(dev)
        o = torch.empty((wl.q_rows, wl.num_heads, wl.head_dim), dtype=torch.float32, device=dev)
        lse = torch.empty((wl.q_rows, wl.num_heads), dtype=torch.float32, device=dev)
        ws = (torch.empty(built.workspace_floats, dtype=torch.float32, device=dev)
              if built.workspace_floats else None)

        def fwd():
            zl.coalesced_attn_fwd(built, q, k, v, o, lse, stream=stream, workspace=ws)

        for _ in range(3):
            fwd()
        torch.cuda.synchronize()
        probe = _events_ms(fwd, 2, stream)
        n = max(5, min(20, int(600.0 / max(probe, 1e-3))))
        sp = _spread(_launch_ms(fwd, n, stream))
        F = wl.flops_fwd()
        rec = {"workload": wl.name, "kv_chunk": kv_chunk, "flops": F, "tiles": built.n_tiles, **sp,
               "TFLOP/s": round(F / (sp["ms_median"] * 1e-3) / 1e12, 2),
               "frac": round(F / (sp["ms_median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        if c == 0:
            rec = {"workload": wl.name, "kv_chunk": kv_chunk, "flops": F, "tiles": built.n_tiles,
                   "us_median": round(1e3 * sp["ms_median"], 2), "us_min": round(1e3 * sp["ms_min"], 2),
                   "launches": sp["launches"]}
        for m in wl.merges:  # the theta-k merge of the partials, after the forward
            mo = torch.empty((m.rows, wl.num_heads, wl.head_dim), dtype=torch.float32, device=dev)
            ml = torch.empty((m.rows, wl.num_heads), dtype=torch.float32, device=dev)

            def step():
                fwd()
                zl.merge_partials(o, lse, m.row0, m.n_parts, m.rows, m.part_row_stride,
                                  m.head_begin, m.head_cnt, mo, ml, stream=stream)

            step()
            torch.cuda.synchronize()
            spm = _spread(_launch_ms(step, n, stream))
            if c != 0:
                rec["with_merge"] = {"ms_median": spm["ms_median"], "ms_min": spm["ms_min"],
                                     "TFLOP/s": round(F / (spm["ms_median"] * 1e-3) / 1e12, 2)}
        out[f"{c}" if kv_chunk == 0 else
            f"{c}_kv_chunk_{'auto' if kv_chunk == zl.KV_CHUNK_AUTO else kv_chunk}"] = rec
        del q, k, v, o, lse, ws, built
        torch.cuda.empty_cache()
    return out


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (the multi-GPU "
              "exchanges are design-only)", file=sys.stderr)
        sys.exit(2)
    import torch
    from coalesced_attention_amd import workloads as W
    from coalesced_attention_amd import zl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if a.calibrate_copy:
        n = 1 << 28  # 1 GiB of fp32
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4}), flush=True)
        return
    if a.calibrate_mfma:
        print(json.dumps(_calibrate_mfma(zl)), flush=True)
        return
    wl = W.config(a.config)
    inp = W.make_inputs(wl)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    n_slots = zl.default_slots(0) if a.n_slots < 0 else a.n_slots
    if a.price_table:
        print(json.dumps(_price_table(zl, wl, q, k, v, dev, n_slots)), flush=True)
        return

    t0 = time.perf_counter()
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim,
                              n_slots=n_slots, kv_chunk=a.kv_chunk)
    wl_ms = (time.perf_counter() - t0) * 1e3
    built.to(dev)
    o = torch.empty((wl.q_rows, wl.num_heads, wl.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.q_rows, wl.num_heads), dtype=torch.float32, device=dev)
    ws = (torch.empty(built.workspace_floats, dtype=torch.float32, device=dev)
          if built.workspace_floats else None)
    stream = torch.cuda.current_stream(dev)

    def step():
        zl.coalesced_attn_fwd(built, q, k, v, o, lse, stream=stream, workspace=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps run back to back, with nothing between the launches;
    # a second pass brackets each launch with its own pair of HIP events for
    # the per-launch spread and the kernel time of the roofline
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    launch_ms = _launch_ms(step, a.steps, stream)
    sp = _spread(launch_ms)
    kern_ms = sp["ms_mean"]

    flops = wl.flops_fwd()
    tflops = flops / (ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "items": len(wl.items), "q_rows": wl.q_rows,
                   "kv_rows": wl.kv_rows, "heads": wl.num_heads, "head_dim": wl.head_dim,
                   "tiles": built.n_tiles, "n_slots": n_slots, "flops_per_step": flops,
                   "kv_chunk": a.kv_chunk,
                   "schedule_makespan_over_mean": round(built.header.max_slot_cost * max(1, n_slots)
                                                        / max(1, built.header.total_cost), 4)},
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "launch_ms": sp,
        "tflops_at_median": round(flops / (sp["ms_median"] * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("fwd_kernel<128>"), "kernel": "fwd_kernel<128>",
                     "kernel_ms": round(kern_ms, 4)},
        "worklist_build_ms": round(wl_ms, 3),
    }
    print(f"[bench] headline forward: {sp}", file=sys.stderr, flush=True)
    if not a.no_calib:
        cal = _calibrate_mfma(zl)
        cal["frac_of_random"] = round(achieved / cal["random_bf16"], 4)
        out["mfma_attainable"] = cal

    if not a.no_price and a.config == 2:
        pt = _price_table(zl, wl, q, k, v, dev, n_slots)
        out["price_table"] = {k2: pt[k2] for k2 in ("coalesced_ms", "sum_bucket_launches_ms",
                                                    "sum_single_prices_ms", "coalesced_over_bucket_launches",
                                                    "coalesced_over_single_prices")}
        out["price_table"]["buckets"] = [{k2: r[k2] for k2 in ("q_len", "kv_len", "head_cnt", "count",
                                                               "single_ms", "bucket_ms")}
                                         for r in pt["buckets"]]
        print(f"[bench] price table done", file=sys.stderr, flush=True)

    if not a.no_merge:
        # KV-split merge at its full size: 2 partials x 27450 rows x 12 of 24 heads
        rows, H, d, parts = 27450, 24, 128, 2
        g = torch.Generator(device=dev).manual_seed(3)
        po = torch.randn((parts * rows, H, d), generator=g, device=dev)
        pl = 10 + torch.randn((parts * rows, H), generator=g, device=dev)
        mo = torch.empty((rows, H, d), device=dev)
        ml = torch.empty((rows, H), device=dev)

        def merge():
            zl.merge_partials(po, pl, 0, parts, rows, rows, 0, 12, mo, ml, stream=stream)

        for _ in range(3):
            merge()
        torch.cuda.synchronize()
        msp = _spread(_launch_ms(merge, 20, stream))
        mms = msp["ms_mean"]
        mbytes = (parts + 1) * rows * 12 * (d + 1) * 4
        out["merge"] = {"workload": "kv-split merge, 2 x 27450 rows x 12 heads x 128", "ms": round(mms, 4),
                        "ms_median": msp["ms_median"], "ms_min": msp["ms_min"],
                        "GB/s": round(mbytes / (mms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(mbytes / (mms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                        "bytes": mbytes, "traffic": measured_traffic("merge_kernel<128>")}
        del po, pl, mo, ml
        # a plain device copy of 1 GiB on the same GPU: the HBM rate a
        # streaming kernel attains here, beside the merge's
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        cms = float(np.median(_launch_ms(lambda: dst.copy_(src), 5, stream)))
        copy_gbps = 2 * (1 << 30) / (cms * 1e-3) / 1e9
        out["merge"]["copy_GB/s"] = round(copy_gbps, 1)
        out["merge"]["frac_of_copy"] = round(mbytes / (mms * 1e-3) / 1e9 / copy_gbps, 4)
        del src, dst

    if not a.no_bwd:
        out["backward"] = _bench_backward(zl, W, dev, stream, n_slots)
        print(f"[bench] backward done", file=sys.stderr, flush=True)

    if not a.no_configs:
        out["configs"] = _bench_configs(zl, W, dev, stream, n_slots)
        print(f"[bench] configs done", file=sys.stderr, flush=True)

    if "mfma_attainable" in out:  # every MFMA rate beside this GPU's random-operand ceiling
        ceil = out["mfma_attainable"]["random_bf16"]
        if "backward" in out:
            out["backward"]["frac_of_random"] = round(out["backward"]["TFLOP/s"] / ceil, 4)
        for rec in out.get("configs", {}).values():
            if "TFLOP/s" in rec:
                rec["frac_of_random"] = round(rec["TFLOP/s"] / ceil, 4)

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(wl, inp, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
