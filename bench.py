#!/usr/bin/env python3
"""Decode-step benchmark of the page-summary hot path on one MI355X.

One step = one layer's decode step as a replayed HIP graph: summary scan +
page-mass aggregation, top-k page selection, sparse paged flash-decode over
the selected pages (+ partial last pages) and the LSE merge.  Inputs are
resident in HBM before timing.  Layer copies are rotated so that repeated
steps do not hit in the 256 MB Infinity Cache.

Also measured in the same run: the summary-scan kernel alone (the dominant
kernel, for the roofline), the dense paged flash-decode baseline (speedup),
the summary build (prefill-time throughput), and the CPU oracle on a bounded
sample (cpu_baseline).

Prints ONE JSON line.  Default workload: GLM-4-9B-shaped layer, 1M tokens,
r = 8, budget 2048 (the headline configuration).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/decode step at 1M ctx r=8 + HBM GB/s (% peak); speedup vs dense decode"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--layers", type=int, default=0, help="layer copies rotated (0 = auto)")
    ap.add_argument("--budget", type=int, default=0, help="override the token budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-bf16-summaries", action="store_true",
                    help="skip the extra measurements of the step with bf16 and with "
                         "int8/int4 summaries")
    ap.add_argument("--cpu-target-s", type=float, default=12.0,
                    help="approximate CPU seconds spent on the oracle sample")
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# Kernel sources whose HBM traffic the committed counter summary describes.
SCAN_SOURCES = ["kv_cache_page_rank_amd/csrc/scan_kernel.hpp",
                "kv_cache_page_rank_amd/csrc/scan_common.hpp",
                "kv_cache_page_rank_amd/csrc/scan_batch_f32.hpp",
                "kv_cache_page_rank_amd/csrc/scan_f32.hip",
                "kv_cache_page_rank_amd/csrc/device_common.hpp",
                "kv_cache_page_rank_amd/csrc/launchers.hpp"]
SCAN_COUNTERS = "profiles/scan_kernel_glm4-9b-layer-1m_hbm_counters.txt"


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_traffic(summary, sources, workload_name):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the copy calibration), or None
    when there is none for this workload or the kernel's sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, summary)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("workload") != workload_name or kv.get("source_sha256") != sources_sha256(sources):
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(args):
    """A plain device-to-device copy of 1 GiB, repeated: under rocprofv3
    --pmc its FETCH_SIZE / WRITE_SIZE per dispatch against the known 1 GiB
    read and 1 GiB written give the counters' scale factors."""
    import torch

    n = 1 << 28  # fp32 elements = 1 GiB
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(1, args.steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                      "dispatches": max(1, args.steps)}), flush=True)


def time_events(fn, iters, torch):
    """Average device time per call of fn() over `iters` calls, each bracketed
    by events on the current stream (the stream the library launches on)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return statistics.mean(ms) * 1e3, statistics.median(ms) * 1e3, ms


def dist(us, per=1):
    """mean / median / p10 / p90 of a list of microseconds (each the mean
    of `per` back-to-back calls)."""
    import numpy as np
    a = np.asarray(us, np.float64)
    return {"samples": int(a.size), "calls_per_sample": per, "replays": int(a.size) * per,
            "mean_us": round(float(a.mean()), 3), "median_us": round(float(np.median(a)), 3),
            "p10_us": round(float(np.percentile(a, 10)), 3),
            "p90_us": round(float(np.percentile(a, 90)), 3)}


def time_samples(fn, samples, per, torch):
    """`samples` timings, each the mean of `per` back-to-back calls between
    two events on the current stream (events only between batches, so their
    own cost is spread over `per` calls).  Returns the dist() record."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    ev[0].record()
    n = 0
    for s_ in range(samples):
        for _ in range(per):
            fn(n)
            n += 1
        ev[s_ + 1].record()
    torch.cuda.synchronize()
    return dist([ev[i].elapsed_time(ev[i + 1]) * 1e3 / per for i in range(samples)], per)


def time_batch(fn, iters, torch):
    """Average device time per call over `iters` back-to-back calls between
    two events on the current stream (no event between calls; the figure
    includes the dispatch gap between consecutive kernels)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is measured on one GPU; sharding over GPUs is not built).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args)
        return

    import numpy as np
    import torch

    import kv_cache_page_rank_amd as lk
    import workload
    from kv_cache_page_rank_amd import traffic
    from workload.device import upload

    if not os.path.exists(lk.LIB_PATH):
        from kv_cache_page_rank_amd import build as _b
        _b.build()
    lk.lib()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")

    spec = workload.config(args.config)
    if args.budget:
        spec = spec.with_(budget_tokens=args.budget)
    threads = args.threads or cpu_threads()
    t0 = time.time()
    layer = workload.make(spec, threads=threads)
    log(f"generated {spec.name} in {time.time() - t0:.1f}s")
    q, kv0, pages = upload(layer, "cuda")
    B, Hq, Hkv, d, P, r = (spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                           spec.page_size, spec.rank)
    NB, MP, k = spec.num_blocks, spec.max_pages, spec.k_pages
    full = [n // P for n in spec.seq_lens]
    partial = sum(1 for n in spec.seq_lens if n % P)
    full_total = sum(full)

    # layer copies: summary + K/V working set per copy; rotate beyond 2 x 256 MB of MALL
    sum_bytes = NB * Hkv * traffic.summary_unit_bytes(d, P, r)
    L = args.layers or max(1, min(8, math.ceil(2 * 256e6 / max(sum_bytes, 1)) + 1))
    kvs = [kv0] + [lk.PagedKV(kv0.k.clone(), kv0.v.clone()) for _ in range(L - 1)]
    summs = [lk.Summaries.empty(NB, Hkv, P, d, r) for _ in range(L)]

    # --- build (prefill-time summary construction), timed on layer 0
    torch.cuda.synchronize()
    bstart, bend = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bstart.record()
    lk.locks_build_summaries(kvs[0], pages, summs[0])
    bend.record()
    torch.cuda.synchronize()
    build_ms = bstart.elapsed_time(bend)
    for i in range(1, L):
        lk.locks_build_summaries(kvs[i], pages, summs[i])
    torch.cuda.synchronize()
    log(f"built {full_total * Hkv} page summaries in {build_ms:.2f} ms (x{L} layers)")

    # --- page-crossing refresh: the last full page of every sequence (what a
    # decode step that completes a page rebuilds), B x H_kv units
    last = torch.tensor([max(n // P - 1, 0) for n in spec.seq_lens], dtype=torch.int32,
                        device="cuda")
    for _ in range(2):
        lk.locks_refresh_summaries(kvs[0], pages, last, 1, summs[0])
    refresh_us = time_batch(lambda i: lk.locks_refresh_summaries(kvs[0], pages, last, 1, summs[0]),
                            5, torch)
    log(f"one-page refresh ({B * Hkv} units): {refresh_us:.1f} us")

    # --- one step graph per layer copy
    ws_step = lk.workspace_bytes(lk.OP_STEP, B, MP, Hq, Hkv, P, d, r, k)
    bufs = []
    graphs = []
    for i in range(L):
        sel = torch.empty((B, Hkv, k), dtype=torch.int32, device="cuda")
        mass = torch.empty((B, Hkv, k), device="cuda")
        out = torch.empty((B, Hq, d), dtype=kv0.k.dtype, device="cuda")
        lse = torch.empty((B, Hq), device="cuda")
        ws = lk.workspace(ws_step)
        bufs.append((sel, mass, out, lse, ws))
        graphs.append(lk.StepGraph(q, summs[i], kvs[i], pages, spec.budget_tokens, sel, mass, out,
                                   lse, ws=ws))

    for i in range(args.warmup):
        graphs[i % L].launch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % L].launch()
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    step_us = e0.elapsed_time(e1) * 1e3 / args.steps
    log(f"step: {step_us:.2f} us (graph replay, {L} layer copies), wall {wall_s * 1e6 / args.steps:.2f} us")
    # the step's distribution: 50 samples, each the mean of 10 back-to-back
    # replays (an event between samples only: one per replay would add its
    # own few microseconds to every replay)
    step_dist = time_samples(lambda i: graphs[i % L].launch(), 50, 10, torch)
    log(f"step over {step_dist['replays']} replays: median {step_dist['median_us']:.2f} us, "
        f"p10 {step_dist['p10_us']:.2f}, p90 {step_dist['p90_us']:.2f}")

    # --- the page-crossing refresh off the step's path: 10 step replays on the
    # launch stream while a one-page refresh (B x H_kv units) runs on a side
    # stream, against 10 replays alone (same graphs; the refresh rewrites the
    # same values, so the overlap only shares the machine)
    side = torch.cuda.Stream()
    n_ov = 10

    def replays(with_refresh):
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        if with_refresh:
            side.wait_stream(torch.cuda.current_stream())
            lk.locks_refresh_summaries(kvs[0], pages, last, 1, summs[0], stream=side)
        for i in range(n_ov):
            graphs[i % L].launch()
        a1.record()
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) * 1e3 / n_ov

    replays(True)
    alone_us = min(replays(False) for _ in range(3))
    overlap_us = min(replays(True) for _ in range(3))
    log(f"step beside a concurrent one-page refresh: {overlap_us:.2f} us per step over {n_ov} "
        f"replays ({alone_us:.2f} alone; the refresh itself takes {refresh_us:.1f} us)")

    # --- dominant kernel: the summary scan alone, per-launch events on the launch stream
    pms = [torch.empty((B, Hkv, MP), device="cuda") for _ in range(L)]
    for i in range(args.warmup):
        lk.locks_scan(q, summs[i % L], pages, pms[i % L])
    scan_ev_mean, scan_med, _ = time_events(
        lambda i: lk.locks_scan(q, summs[i % L], pages, pms[i % L]), args.steps, torch)
    # the roofline's launch duration: back-to-back launches between two
    # events (per-launch event pairs add their own ~1-2 us to every launch)
    scan_mean = time_batch(lambda i: lk.locks_scan(q, summs[i % L], pages, pms[i % L]),
                           args.steps, torch)
    scan_b = traffic.scan_bytes(B, Hq, Hkv, MP, full_total, d, P, r)
    scan_dist = time_samples(lambda i: lk.locks_scan(q, summs[i % L], pages, pms[i % L]), 50,
                             10, torch)
    # the roofline's average launch duration: the mean over all 500 sampled
    # back-to-back launches (the K-launch figure above is kept beside it)
    scan_k = scan_mean
    scan_mean = scan_dist["mean_us"]
    scan_gbs = scan_b / (scan_mean * 1e-6) / 1e9
    log(f"scan: {scan_mean:.2f} us per launch back to back over 500 launches ({scan_k:.2f} over "
        f"{args.steps}; {scan_ev_mean:.2f} mean, "
        f"{scan_med:.2f} median with an event pair per launch; median of 10-launch means "
        f"{scan_dist['median_us']:.2f}), {scan_gbs:.0f} GB/s")

    # --- ceilings measured with the same build: a contiguous streaming read of
    # 4 GiB, and the scan's own bytes read in its access pattern with none of
    # its arithmetic (fp32 summaries at P 64, d 128, r 8)
    ceilings = {}
    sbuf = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    sbuf.fill_(1.0)
    sink = torch.empty(4 * 16384, dtype=torch.float32, device="cuda")
    best = (0.0, 0)
    for blocks in (1024, 2048, 4096, 8192, 16384):  # the best grid is the ceiling
        sk = sink[:4 * blocks]
        for _ in range(2):
            lk.locks_probe_stream_read(sbuf, sk)
        st_us = time_batch(lambda i: lk.locks_probe_stream_read(sbuf, sk), 10, torch)
        gbs = sbuf.numel() * 4 / (st_us * 1e-6) / 1e9
        log(f"ceiling: streaming read of 4 GiB, {blocks} workgroups: {st_us:.1f} us, "
            f"{gbs:.0f} GB/s")
        best = max(best, (gbs, blocks))
    ceilings["stream_read_GBps"] = round(best[0], 1)
    ceilings["stream_read_workgroups"] = best[1]
    ceilings["stream_read_bytes"] = sbuf.numel() * 4
    del sbuf
    if (P, d, r) == (64, 128, 8):
        for i in range(args.warmup):
            lk.locks_probe_summary_read(q, summs[i % L], pages, pms[i % L])
        pat_us = time_samples(lambda i: lk.locks_probe_summary_read(q, summs[i % L], pages,
                                                                     pms[i % L]), 50, 10,
                              torch)["mean_us"]
        pat_gbs = scan_b / (pat_us * 1e-6) / 1e9
        ceilings.update({"scan_pattern_read_us": round(pat_us, 3),
                         "scan_pattern_read_GBps": round(pat_gbs, 1)})
        log(f"ceiling: the scan's bytes in its access pattern {pat_us:.2f} us, {pat_gbs:.0f} GB/s")
    torch.cuda.empty_cache()

    # --- select alone and sparse attention alone
    sel_ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, B, MP, Hq, Hkv, P, d, r, k))
    sel_mean, _, _ = time_events(
        lambda i: lk.locks_select(q, summs[i % L], pages, spec.budget_tokens, bufs[i % L][0],
                                  bufs[i % L][1], ws=sel_ws), args.steps, torch)
    att_ws = lk.workspace(lk.workspace_bytes(lk.OP_SPARSE_ATTEND, B, MP, Hq, Hkv, P, d, r, k))
    sparse_mean, _, _ = time_events(
        lambda i: lk.locks_sparse_attend(q, kvs[i % L], pages, bufs[i % L][0], bufs[i % L][2],
                                         bufs[i % L][3], ws=att_ws), args.steps, torch)
    # the same calls back to back (attention kernel + merge kernel per call), and
    # the K/V bytes they must read: the selected pages and the partial last pages
    sparse_b2b = time_batch(
        lambda i: lk.locks_sparse_attend(q, kvs[i % L], pages, bufs[i % L][0], bufs[i % L][2],
                                         bufs[i % L][3], ws=att_ws), args.steps, torch)
    sparse_b = (B * Hkv * k + partial * Hkv) * traffic.kv_unit_bytes(d, P)
    step_b = traffic.step_bytes(full_total, partial, Hkv, d, P, r, B * Hkv * k)
    log(f"select (scan+topk): {sel_mean:.2f} us, sparse attend+merge: {sparse_mean:.2f} us "
        f"({sparse_b2b:.2f} us back to back, {sparse_b / (sparse_b2b * 1e-6) / 1e9:.0f} GB/s)")

    # --- the same step with reduced-precision summaries (reported beside the
    # fp32 headline): bf16 values, and the pages' own int8 / int4 codes.  The
    # summaries get enough rotated copies that every copy's reuse distance
    # exceeds 2 x 256 MB (the K/V copies rotate as before).
    def reduced_precision(dtype, elem, label):
        scan_b = traffic.scan_bytes(B, Hq, Hkv, MP, full_total, d, P, r, summary_elem=elem)
        n = max(L, -(-2 * 256 * 2 ** 20 // scan_b) + 1)
        copies = [lk.Summaries.empty(NB, Hkv, P, d, r, dtype=dtype) for _ in range(n)]
        for i in range(n):
            lk.locks_build_summaries(kvs[i % L], pages, copies[i])
        graphs = [lk.StepGraph(q, copies[i], kvs[i % L], pages, spec.budget_tokens,
                               *bufs[i % L][:4], ws=bufs[i % L][4]) for i in range(n)]
        for i in range(max(args.warmup, n)):
            graphs[i % n].launch()
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            graphs[i % n].launch()
        e1.record()
        torch.cuda.synchronize()
        step_us = e0.elapsed_time(e1) * 1e3 / args.steps
        for i in range(max(args.warmup, n)):
            lk.locks_scan(q, copies[i % n], pages, pms[i % L])
        scan_us = time_batch(lambda i: lk.locks_scan(q, copies[i % n], pages, pms[i % L]),
                             args.steps, torch)
        gbs = scan_b / (scan_us * 1e-6) / 1e9
        for g_ in graphs:
            g_.close()
        log(f"{label}: step {step_us:.2f} us, scan {scan_us:.2f} us, {gbs:.0f} GB/s "
            f"({n} summary copies)")
        return {"step_us": round(step_us, 3), "scan_us": round(scan_us, 3),
                "scan_bytes_per_launch": scan_b, "scan_GBps": round(gbs, 1),
                "scan_frac": round(gbs / HBM_PEAK_GBS, 4), "summary_copies": n,
                "speedup_vs_dense": None,
                "summary_to_cache_ratio": round(traffic.summary_to_cache_ratio(d, P, r, elem), 4)}

    bf16_summ = q8q4_summ = None
    if not args.no_bf16_summaries:
        bf16_summ = reduced_precision(torch.bfloat16, 2, "bf16 summaries")
        q8q4_summ = reduced_precision(lk.Q8Q4, "q8q4", "int8/int4 summaries")

    # --- the same step with the mean-of-share group aggregation (fp32 summaries)
    gm = [lk.StepGraph(q, summs[i], kvs[i], pages, spec.budget_tokens, *bufs[i][:4], ws=bufs[i][4],
                       agg=lk.AGG_MEAN_SHARE) for i in range(L)]
    for i in range(args.warmup):
        gm[i % L].launch()
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        gm[i % L].launch()
    e1.record()
    torch.cuda.synchronize()
    share_step = e0.elapsed_time(e1) * 1e3 / args.steps
    for g_ in gm:
        g_.close()
    log(f"mean-of-share aggregation: step {share_step:.2f} us")

    # --- dense baseline
    dense_mean = dense_dist = None
    dense_b = traffic.dense_bytes(sum(-(-n // P) for n in spec.seq_lens), Hkv, d, P)
    if not args.no_dense:
        dws = lk.workspace(lk.workspace_bytes(lk.OP_DENSE_ATTEND, B, MP, Hq, Hkv, P, d, r, 0))
        dout = torch.empty((B, Hq, d), dtype=kv0.k.dtype, device="cuda")
        dlse = torch.empty((B, Hq), device="cuda")
        for i in range(2):
            lk.locks_dense_attend(q, kvs[i % L], pages, dout, dlse, ws=dws)
        dense_dist = time_samples(
            lambda i: lk.locks_dense_attend(q, kvs[i % L], pages, dout, dlse, ws=dws), 50, 4,
            torch)
        dense_mean = dense_dist["mean_us"]
        log(f"dense: {dense_mean:.2f} us (median {dense_dist['median_us']:.2f}), "
            f"{dense_b / (dense_mean * 1e-6) / 1e9:.0f} GB/s")
        for rp in (bf16_summ, q8q4_summ):
            if rp is not None:
                rp["speedup_vs_dense"] = round(dense_mean / rp["step_us"], 3)

    # --- CPU baseline: the oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, layer, target_s=args.cpu_target_s, threads=threads)

    ratio = traffic.summary_to_cache_ratio(d, P, r)
    result = {
        "metric": METRIC,
        "value": round(step_us, 3),
        "unit": "µs/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "page_size": P, "context_tokens": spec.seq_lens
                   if B > 1 else spec.seq_lens[0], "rank": r, "budget_tokens": spec.budget_tokens,
                   "kv_dtype": "bf16" if spec.kv_bf16 else "f32", "summary_dtype": "f32",
                   "layer_copies_rotated": L, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "summary scan",
                     "achieved": round(scan_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic(SCAN_COUNTERS, SCAN_SOURCES, spec.name),
                     "bytes_per_launch": scan_b, "avg_launch_us": round(scan_mean, 3),
                     "avg_launch_us_k_launches": round(scan_k, 3),
                     "avg_launch_us_event_pairs": round(scan_ev_mean, 3),
                     "launch_dist": scan_dist, "ceilings": ceilings,
                     "frac_of_stream_ceiling": round(scan_gbs / ceilings["stream_read_GBps"], 4),
                     "frac_of_pattern_ceiling": None if "scan_pattern_read_GBps" not in ceilings
                     else round(scan_gbs / ceilings["scan_pattern_read_GBps"], 4)},
        "cpu_baseline": cpu,
        "step_dist": step_dist,
        "breakdown": {
            "scan_us": round(scan_mean, 3),
            "select_us": round(sel_mean, 3),
            "sparse_attend_us": round(sparse_mean, 3),
            "sparse_attend_back_to_back_us": round(sparse_b2b, 3),
            "sparse_attend_bytes": sparse_b,
            "sparse_attend_GBps": round(sparse_b / (sparse_b2b * 1e-6) / 1e9, 1),
            "dense_attend_us": None if dense_mean is None else round(dense_mean, 3),
            "dense_dist": dense_dist,
            "speedup_vs_dense": None if dense_mean is None else round(dense_mean / step_us, 3),
            "speedup_vs_dense_medians": None if dense_dist is None else
            round(dense_dist["median_us"] / step_dist["median_us"], 3),
            "step_bytes": step_b,
            "dense_bytes": dense_b,
            "byte_reduction": round(dense_b / step_b, 3),
            "step_GBps": round(step_b / (step_us * 1e-6) / 1e9, 1),
            "dense_GBps": None if dense_mean is None else
            round(dense_b / (dense_mean * 1e-6) / 1e9, 1),
            "summary_to_cache_ratio": round(ratio, 4),
            "build_ms": round(build_ms, 3),
            "build_pages_per_s": round(full_total * Hkv / (build_ms * 1e-3), 1),
            "refresh_one_page_us": round(refresh_us, 1),
            "step_beside_refresh_us": round(overlap_us, 3),
            "step_alone_same_window_us": round(alone_us, 3),
            "bf16_summaries": bf16_summ,
            "q8q4_summaries": q8q4_summ,
            "mean_share_step_us": round(share_step, 3),
        },
    }
    for g in graphs:
        g.close()
    print(json.dumps(result), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, layer, target_s, threads):
    """Time the oracle on the host cores, on the same layer.

    The decode step: scan + aggregation over every full page, selection from
    those masses, and attention over the pages it selected - with all
    `threads` cores (repeated for about target_s seconds) and with one thread
    (a few repeats).  Nothing here comes from the GPU: the summaries are
    seeded stand-ins of the layer's shapes (the oracle's cost does not depend
    on their values).  When one step alone is longer than target_s, a prefix
    of the pages is scanned and the time scaled to all pages.

    The summary build (the oracle's one-sided Jacobi SVD of every page), on a
    prefix of the pages (all KV heads), with all cores and with one thread,
    extrapolated per unit to every full page of the layer; dense attention
    over a prefix of every sequence, scaled per token.  Returns the JSON
    record."""
    import numpy as np

    import oracle

    P, Hkv, d, r = spec.page_size, spec.num_kv_heads, spec.head_dim, spec.rank
    g = np.random.default_rng(spec.seed + 17)
    NB = spec.num_blocks
    mu = g.standard_normal((NB, Hkv, d), dtype=np.float32)
    basis = g.standard_normal((NB, Hkv, r, d), dtype=np.float32) / np.float32(np.sqrt(d))
    coef = g.standard_normal((NB, Hkv, P, r), dtype=np.float32)
    full_total = sum(n // P for n in spec.seq_lens)
    kf, vf = layer.k_f32(), layer.v_f32()  # widened once, outside the timed calls
    lay_full = oracle.Layout(spec.num_q_heads, Hkv, d, P, layer.block_table, layer.seq_lens)

    def step(npages, nthreads):
        """Scan + selection over the first npages full pages of each sequence."""
        seq = np.array([min(n, npages * P) for n in spec.seq_lens], np.int32)
        lay = oracle.Layout(spec.num_q_heads, Hkv, d, P, layer.block_table, seq)
        t0 = time.perf_counter()
        _, pm = oracle.scan_pool(lay, r, layer.q, mu, basis, coef, threads=nthreads, heads=False)
        t1 = time.perf_counter()
        sel, _ = oracle.select_pool(lay, spec.budget_tokens, pm.astype(np.float32), spec.k_pages)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1, int(sum(s // P for s in seq)), sel

    def timed_step(nthreads, budget_s, max_reps):
        npages = max(full_total, 1)
        scan_s, sel_s, done, sel = step(npages, nthreads)
        t0 = time.perf_counter()
        oracle.attend_pool(lay_full, layer.q, kf, vf, sel, threads=nthreads)
        att_s = time.perf_counter() - t0
        if scan_s + sel_s + att_s > budget_s:  # one step is already long: scan a prefix
            npages = max(1, int(npages * budget_s / (scan_s + sel_s + att_s)))
            scan_s, sel_s, done, _ = step(npages, nthreads)
            scan_s *= full_total / max(done, 1)
            return scan_s, sel_s, att_s, (f"scan+aggregation+selection over the first {done} of "
                                          f"{full_total} full pages (x{Hkv} KV heads), scaled "
                                          f"to all pages; attention over the selected pages")
        reps = max(1, min(max_reps, int(budget_s / (scan_s + sel_s + att_s))))
        tot_scan = tot_sel = tot_att = 0.0
        for _ in range(reps):
            a, s_, _, sel = step(npages, nthreads)
            t0 = time.perf_counter()
            oracle.attend_pool(lay_full, layer.q, kf, vf, sel, threads=nthreads)
            tot_att += time.perf_counter() - t0
            tot_scan += a
            tot_sel += s_
        return (tot_scan / reps, tot_sel / reps, tot_att / reps,
                f"the full step (scan+aggregation over all {full_total} full pages x{Hkv} KV "
                f"heads, selection, attention over the selected pages), mean of {reps} repeats")

    scan_s, sel_s, att_s, sample = timed_step(threads, 0.6 * target_s, 10 ** 6)
    step_s = scan_s + sel_s + att_s
    log(f"cpu oracle: scan {scan_s * 1e3:.1f} ms, select {sel_s * 1e3:.1f} ms, attend "
        f"{att_s * 1e3:.1f} ms -> {step_s * 1e6:.0f} us/step on {threads} threads ({sample})")
    s1, se1, a1, sample1 = timed_step(1, 0.2 * target_s, 5)
    step1_s = s1 + se1 + a1
    log(f"cpu oracle, one thread: {step1_s * 1e6:.0f} us/step ({sample1})")

    # summary build on a prefix of each sequence's pages, every KV head
    def build_sample(nthreads, npages):
        seq = np.array([min(n, npages * P) for n in spec.seq_lens], np.int32)
        lay = oracle.Layout(spec.num_q_heads, Hkv, d, P, layer.block_table, seq)
        units = int(sum(s_ // P for s_ in seq)) * Hkv
        t0 = time.perf_counter()
        oracle.build_pool(lay, r, kf, NB, threads=nthreads)
        return time.perf_counter() - t0, units

    ball_s, ball_u = build_sample(threads, max(1, 64 * threads // (Hkv * spec.batch)))
    b1_s, b1_u = build_sample(1, max(1, 48 // (Hkv * spec.batch)))
    all_units = full_total * Hkv
    build_all_ms = ball_s / ball_u * all_units * 1e3
    build_one_ms = b1_s / b1_u * all_units * 1e3
    log(f"cpu oracle build: {ball_u} units in {ball_s:.2f} s on {threads} threads, {b1_u} units "
        f"in {b1_s:.2f} s on one thread -> {all_units} units: {build_all_ms / 1e3:.1f} s / "
        f"{build_one_ms / 1e3:.1f} s (extrapolated per unit)")
    # dense attention (every token of every sequence) on a prefix of each
    # sequence sized to about a second, scaled per token to the whole layer
    def dense_sample(nthreads, ntok):
        seq = np.array([min(n, ntok) for n in spec.seq_lens], np.int32)
        lay = oracle.Layout(spec.num_q_heads, Hkv, d, P, layer.block_table, seq)
        t0 = time.perf_counter()
        oracle.attend_pool(lay, layer.q, kf, vf, None, threads=nthreads)
        return time.perf_counter() - t0, int(seq.sum())

    all_tokens = int(sum(spec.seq_lens))

    def dense_timed(nthreads, budget_s):
        ntok = 16 * P
        s_, done = dense_sample(nthreads, ntok)
        while s_ < 0.25 * budget_s and done < all_tokens:
            ntok = ntok * max(2, min(64, int(0.5 * budget_s / max(s_, 1e-4))))
            s_, done = dense_sample(nthreads, ntok)
        return s_ / done * all_tokens * 1e3, done

    dense_all_ms, dense_all_tok = dense_timed(threads, 0.1 * target_s)
    dense_one_ms, dense_one_tok = dense_timed(1, 0.1 * target_s)
    log(f"cpu oracle dense attention: {dense_all_ms:.1f} ms on {threads} threads "
        f"({dense_all_tok} tokens timed), {dense_one_ms:.1f} ms on one thread ({dense_one_tok} "
        f"tokens timed), per step over {all_tokens} tokens")
    return {"value": round(step_s * 1e6, 1), "unit": "µs/step", "cores": threads,
            "kind": "oracle", "sample": sample, "cpu_model": cpu_model(),
            "one_thread": {"value": round(step1_s * 1e6, 1), "unit": "µs/step", "cores": 1,
                           "sample": sample1},
            "build": {"all_cores_ms_extrapolated": round(build_all_ms, 1),
                      "one_thread_ms_extrapolated": round(build_one_ms, 1),
                      "units": all_units,
                      "sample": f"oracle build of {ball_u} units on {threads} threads and "
                                f"{b1_u} units on one thread (the first pages of each "
                                f"sequence, every KV head), scaled per unit"},
            "dense_attend": {"all_cores_ms": round(dense_all_ms, 2),
                             "one_thread_ms": round(dense_one_ms, 2),
                             "sample": f"dense attention over the first {dense_all_tok} tokens "
                                       f"({threads} threads) and {dense_one_tok} tokens (one "
                                       f"thread) of the sequences, scaled per token to all "
                                       f"{all_tokens}"}}


if __name__ == "__main__":
    main()
