#!/usr/bin/env python3
"""Benchmark: one decode step of the FP4 lightning indexer at 1M context on one MI355X.

Workload ("fullscan_1m"): 8 sequences x 2^20 visible compressed keys (decoder, m = 1), one
query each, 32 heads x 128 dims, MXFP4 queries and keys, synthetic seeded inputs. One step is the
whole hot path for that batch: quantise the Full layer's queries, scan every key (block-8
maxima fused), build the candidate pool (pin + top-2048 blocks), take the Full layer's top-512,
then 4 Reindex layers (quantise their queries, gather-score the pool, top-512 each).

Prints one JSON line: entries scored per second over the step (Full-layer keys + pooled keys of
the Reindex layers), top-512 queries per second, the scan kernel's HBM roofline fraction
(achieved from HIP events around the scan launches of the timed steps), and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def scan_bytes(n_vis, nq: int) -> int:
    """algorithmic bytes of one scan launch: 68 B per key, q (32 x 68 B) + w (128 B) per query,
    4 B per block maximum written"""
    keys = int(sum(n_vis))
    blocks = int(sum((n + 7) // 8 for n in n_vis))
    return keys * 68 + nq * (32 * 68 + 32 * 4) + blocks * 4


def measured_traffic(record: str) -> int | None:
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter record
    (profiles/<record>.json), or None when the kernel's sources have changed since the counters
    were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", record + ".json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return int(rec["traffic_bytes_per_launch"]) if h.hexdigest() == rec["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(wl, max_queries: int = 8, max_keys: int = 1 << 19) -> dict:
    """The oracle (plain C, threaded over queries) on a bounded sample: the Full layer of the
    first min(8, cores) queries of the same workload (score every visible key, top-512, block
    maxima, pin, pool), each over its first min(n, 2^19) visible keys so that the sample stays
    within tens of seconds on slow hosts. The oracle quantises those keys first (untimed)."""
    import numpy as np

    import oracle

    cores = os.cpu_count() or 1
    nqs = max(1, min(max_queries, wl.nq, cores))
    s = wl.signs()
    seqs = sorted(set(int(b) for b in wl.qseq[:nqs]))
    log(f"cpu baseline: oracle quantises the keys of {len(seqs)} sequence(s) (untimed)")
    kcs, kss, seq_off, off = [], [], {}, 0
    for b in seqs:
        kc, ks = oracle.quantize(wl.keys(b, 0, min(int(wl.seq_len[b]), max_keys)), s, nthreads=cores)
        kcs.append(kc)
        kss.append(ks)
        seq_off[b] = off
        off += kc.shape[0]
    kc = np.concatenate(kcs)
    ks = np.concatenate(kss)
    qc, qs = oracle.quantize(wl.q(0, range(nqs)), s)
    w = wl.w(0, range(nqs))
    n = np.minimum(wl.n_vis[:nqs].astype(np.int64), max_keys)
    base = np.array([seq_off[int(b)] for b in wl.qseq[:nqs]], dtype=np.int64)
    log(f"cpu baseline: timing the oracle Full layer on {nqs} queries with {nqs} threads")
    t0 = time.perf_counter()
    oracle.decode_batch(kc, ks, base, n, qc, qs, w, k=wl.k, nthreads=nqs)
    dt = time.perf_counter() - t0
    entries = int(n.sum())
    return {"value": entries / dt, "unit": "entries/s", "cores": nqs, "kind": "oracle",
            "sample": f"Full layer (score all keys, top-512, block max, pin, top-2048 pool) of {nqs} of the "
                      f"{wl.nq} queries, each over its first {int(n[0])} visible keys; {dt:.2f} s wall on "
                      f"{nqs} threads",
            "seconds": round(dt, 3)}


MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak, published


def bench_prefill(wl, args) -> int:
    """Chunked prefill: 4096 consecutive queries on 131072 keys, causal; the step is quantise q,
    the many-query scan (block maxima), top-512 blocks per query, re-score of those 4096 keys,
    final top-512. The roofline is the scan's FP4 matrix throughput."""
    import numpy as np
    import torch

    from top_fp4_lightning_amd import pipeline

    t = time.perf_counter()
    dev = pipeline.DeviceWorkload.from_workload(wl, group=wl.nq)
    torch.cuda.synchronize()
    log(f"workload {wl.name}: {wl.nq} queries, {wl.total_keys} keys; setup {time.perf_counter() - t:.1f} s")
    plan = pipeline.PrefillPlan(dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        plan.run(events=evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / args.steps
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    pairs = int(wl.n_vis.sum())
    flop = 2.0 * 4096.0 * pairs
    achieved = flop / (scan_ms / 1000.0) / 1e12
    print(json.dumps({
        "metric": "prefill (query, key) pairs scored/s; % of FP4 MFMA roofline",
        "value": pairs / (ms_step / 1000.0), "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "prefill_128k: 4096 queries x 131072 keys, causal (query i sees <= 126976+i)"},
        "queries_per_s": wl.nq / (ms_step / 1000.0), "scan_ms": scan_ms,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_FP4_PEAK_TFLOPS,
                     "traffic": measured_traffic("score_multi_prefill_128k_traffic"), "kernel": "score_multi_kernel",
                     "algorithmic_flop_per_launch": flop},
    }), flush=True)
    return 0


DECODE_CONFIGS = {
    "fullscan_1m": "fullscan_1m decode step: batch 8 x 1048576 keys (m=1), Full scan + top-512 + "
                   "pool(2048 blocks of 8) + 4 Reindex layers",
    "spec_decode_1m": "spec_decode_1m verify step: batch 8 x 1048576 keys (m=1), 6 positions per sequence "
                      "(token + 5 draft), Full scan + top-512 + pool(2048 blocks of 8) + 4 Reindex layers",
}


def bench_decode(wl, args) -> int:
    """One decode step per timed iteration (quantise, Full scan, pool, Full top-512 through the
    pool, Reindex layers). With one query per sequence the Full scan is the single-query kernel
    and the roofline is HBM; with several positions per sequence (speculative verification) it is
    the many-query kernel and the roofline is FP4 MFMA."""
    import numpy as np
    import torch

    from top_fp4_lightning_amd import pipeline

    t = time.perf_counter()
    dev = pipeline.DeviceWorkload.from_workload(wl)
    torch.cuda.synchronize()
    log(f"workload {wl.name}: {wl.nq} queries, {wl.total_keys} keys, {wl.layers} Reindex layers; "
        f"setup {time.perf_counter() - t:.1f} s")
    plan = pipeline.DecodePlan(dev)
    stream = torch.cuda.current_stream()

    def step(ev=None, gev=None):
        plan.quantize(0)
        if ev is not None:
            ev[0].record(stream)
        plan.full_scan()
        if ev is not None:
            ev[1].record(stream)
        plan.build_pool()
        plan.pool_select(0, events=gev)
        for layer in range(1, plan.layers + 1):
            plan.quantize(layer)
            plan.pool_select(layer)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    def pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    evs = [pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1000.0 / args.steps
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # The pool gather, timed outside the timed steps. Cold: the Full layer's gather right after
    # the scan, whose stream has replaced the cache contents, so its pooled blocks come from HBM
    # (one event pair per launch, which adds the events' own few microseconds). Warm: the same
    # gather launched back to back between one event pair, its blocks in the last-level cache, as
    # for Reindex layers that follow one another with nothing in between.
    gevs = [pair() for _ in range(args.steps)]
    for i in range(args.steps):
        step(None, gevs[i])
    burst = pair()
    burst[0].record(stream)
    for _ in range(args.steps):
        plan.pool_gather(0)
    burst[1].record(stream)
    torch.cuda.synchronize()
    gather_cold_ms = float(np.mean([a.elapsed_time(b) for a, b in gevs]))
    gather_warm_ms = burst[0].elapsed_time(burst[1]) / args.steps
    ms_eager = ms_step
    if args.graph:
        # the whole step captured once in a HIP graph (the plan allocates nothing and the library
        # issues no memsets) and replayed: no per-launch host work inside the timed region
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            plan.run(stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            plan.run(stream=torch.cuda.current_stream())
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1000.0 / args.steps

    n_vis = [int(x) for x in wl.n_vis]
    pool_pos = int(sum(min(n, 8 * min(2048, (n + 7) // 8)) for n in n_vis))
    entries = int(sum(n_vis)) + plan.layers * pool_pos
    queries = wl.nq * (1 + plan.layers)
    if dev.group == 1:
        sb = scan_bytes(n_vis, wl.nq)
        achieved = sb / (scan_ms / 1000.0) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS,
                    "traffic": measured_traffic("score_full_fullscan_1m_traffic") if wl.name == "fullscan_1m" else None,
                    "kernel": "score_full_kernel", "algorithmic_bytes_per_launch": sb}
    else:
        # many-query scan: keys are read once per group, the matrix work grows with the positions
        flop = 2.0 * 4096.0 * float(sum(n_vis))
        groups = [n_vis[i:i + dev.group] for i in range(0, len(n_vis), dev.group)]
        sb = sum(max(g) * 68 for g in groups) + wl.nq * (32 * 68 + 32 * 4) + sum((n + 7) // 8 for n in n_vis) * 4
        achieved = flop / (scan_ms / 1000.0) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / MFMA_FP4_PEAK_TFLOPS, "traffic": None, "kernel": "score_multi_kernel",
                    "algorithmic_flop_per_launch": flop, "algorithmic_bytes_per_launch": sb,
                    "hbm_achieved_gbs": sb / (scan_ms / 1000.0) / 1e9,
                    "hbm_frac": sb / (scan_ms / 1000.0) / 1e9 / HBM_PEAK_GBS}
    # gather: 68 B per pooled key, q (32 x 68 B) + w (128 B) per query, 4 B per score slot written
    slots = wl.nq * plan.max_blocks * 8
    gb = pool_pos * 68 + wl.nq * (32 * 68 + 32 * 4) + slots * 4
    gather = {"kernel": "score_gather_kernel", "algorithmic_bytes_per_launch": gb,
              "ms_cold": gather_cold_ms, "hbm_frac_cold": gb / (gather_cold_ms / 1000.0) / 1e9 / HBM_PEAK_GBS,
              "ms_warm": gather_warm_ms, "frac_warm": gb / (gather_warm_ms / 1000.0) / 1e9 / HBM_PEAK_GBS,
              "traffic": measured_traffic("score_gather_reindex_1m_traffic") if wl.name == "reindex_1m" else None}
    res = {
        "metric": "indexer entries scored/s + top-512 queries/s at 1M ctx; % of HBM roofline",
        "value": entries / (ms_step / 1000.0),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic (seeded N(0,1) bf16 q/k, N(0,1/32) w, 1% planted keys; no trained weights)",
        "config": {"workload": DECODE_CONFIGS.get(wl.name, wl.name),
                   "batch": wl.nseq, "positions_per_sequence": dev.group, "context": int(wl.seq_len[0]),
                   "reindex_layers": plan.layers, "k": 512, "pool_blocks": 2048, "block": 8},
        "top512_queries_per_s": queries / (ms_step / 1000.0),
        "full_scan_entries_per_s": int(sum(n_vis)) / (scan_ms / 1000.0),
        "scan_ms": scan_ms,
        "step_launch": "hip graph replay" if args.graph else "eager launches",
        "ms_per_step_eager": ms_eager,
        "roofline": roofline,
        "gather": gather,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)
    return 0


def bench_mask_form(args) -> int:
    """The decode step at fullscan_1m in the pool's training form, all 5 layers batched: one
    many-query scan writes every layer's full score row (8 x 5 rows of 2^20), then the pool and a
    top-512 per row over its query's pooled positions ("DeepSeek-V4.1 model structure (3)",
    sections "three details of the pool in the code" and "the pool also acts in training"). Timed
    beside it on the same resident inputs: the literal form (the mask written in place, then a
    top-512 over whole rows) and the gather form (the inference step of bench_decode); all three
    give the same selections. The roofline is the scan's FP4 matrix rate."""
    import numpy as np
    import torch

    import synth
    from top_fp4_lightning_amd import pipeline

    wl = synth.config("fullscan_1m")
    t = time.perf_counter()
    dev = pipeline.DeviceWorkload.from_workload(wl)
    mask = pipeline.MaskFormPlan(dev)
    literal = pipeline.MaskFormPlan(dev, write_mask=True)
    gather = pipeline.DecodePlan(dev)
    torch.cuda.synchronize()
    log(f"mask_form_1m: {wl.nq} queries x {mask.L} layers, {wl.total_keys} keys; setup {time.perf_counter() - t:.1f} s")

    def timed(run, steps, ev=None):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(None if ev is None else ev[i])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / steps

    def mask_step(e=None):
        mask.run(events=e)

    timed(mask_step, args.warmup)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    ms_mask = timed(mask_step, args.steps, evs)
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    timed(lambda e: literal.run(), args.warmup)
    ms_literal = timed(lambda e: literal.run(), args.steps)
    timed(lambda e: gather.run(), args.warmup)
    ms_gather = timed(lambda e: gather.run(), args.steps)
    n_vis = [int(x) for x in wl.n_vis]
    entries = mask.L * int(sum(n_vis))
    flop = 2.0 * 4096.0 * entries
    achieved = flop / (scan_ms / 1000.0) / 1e12
    sb = int(sum(n_vis)) * 68 + mask.rows * (32 * 68 + 32 * 4) + entries * 4 + mask.L * sum((n + 7) // 8 for n in n_vis) * 4
    res = {
        "metric": "indexer entries scored/s + top-512 queries/s at 1M ctx, training form (mask after full scan)",
        "value": entries / (ms_mask / 1000.0), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_mask, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic (seeded N(0,1) bf16 q/k, N(0,1/32) w, 1% planted keys; no trained weights)",
        "config": {"workload": "mask_form_1m: 8 x 1048576 keys, Full + 4 Reindex layers each scoring every "
                               "position in one many-query scan, pool, top-512 per layer over the pooled "
                               "positions", "batch": wl.nseq,
                   "layers": mask.L, "k": 512, "pool_blocks": 2048, "block": 8},
        "top512_queries_per_s": mask.rows / (ms_mask / 1000.0),
        "scan_ms": scan_ms,
        "mask_written_ms_per_step": ms_literal,
        "gather_form_ms_per_step": ms_gather,
        "mask_over_gather": ms_mask / ms_gather,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_FP4_PEAK_TFLOPS, "traffic": None, "kernel": "score_multi_kernel",
                     "algorithmic_flop_per_launch": flop, "algorithmic_bytes_per_launch": sb,
                     "hbm_achieved_gbs": sb / (scan_ms / 1000.0) / 1e9},
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_token(args) -> int:
    """The indexer work of one decode token at 1M context, batch 8: the encoder's 3 Full layers
    (8 x 2^19 keys each, own caches), then the decoder's Full layer (8 x 2^20), pool and 4 Reindex
    layers. Per token 3 x 2.1e9 + 4.3e9 + 2.7e8 = 1.1e10 FP4 MACs ("DeepSeek-V4.1 model structure
    (3)", the per-token totals with the candidate pool)."""
    import numpy as np
    import torch

    import synth
    from top_fp4_lightning_amd import pipeline

    t = time.perf_counter()
    encs, dec = synth.token_1m()
    plan = pipeline.TokenPlan([pipeline.DeviceWorkload.from_workload(w) for w in encs],
                              pipeline.DeviceWorkload.from_workload(dec))
    torch.cuda.synchronize()
    log(f"token_1m: 3 encoder caches of {encs[0].total_keys} keys, decoder {dec.total_keys} keys; "
        f"setup {time.perf_counter() - t:.1f} s")
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan.run()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / args.steps
    nb = dec.nq
    enc_entries = sum(int(w.n_vis.sum()) for w in encs)
    dec_entries = int(dec.n_vis.sum())
    rei_entries = dec.layers * nb * 16384
    entries = enc_entries + dec_entries + rei_entries
    macs = 4096 * entries
    queries = nb * (len(encs) + 1 + dec.layers)
    res = {
        "metric": "indexer entries scored/s + top-512 queries/s for one decode token at 1M ctx (all 8 indexer layers)",
        "value": entries / (ms_step / 1000.0), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic (seeded N(0,1) bf16 q/k, N(0,1/32) w, 1% planted keys; no trained weights)",
        "config": {"workload": "token_1m: batch 8; encoder 3 Full layers x 2^19 keys (m=2, own caches) + decoder "
                               "Full 2^20 + pool(2048 blocks of 8) + 4 Reindex layers", "batch": nb},
        "fp4_macs_per_token": macs / nb,
        "top512_queries_per_s": queries / (ms_step / 1000.0),
        "macs_per_s": macs / (ms_step / 1000.0),
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_kv_gather(args) -> int:
    """Main-KV gather for core attention at the Reindex decode shape: 64 sequences x 2^20
    compressed entries of FP4 main KV resident in HBM (288 bytes each); one step gathers the
    512 selected entries of every query for each of the 5 selections of a decode step (Full +
    4 Reindex layers) and dequantises them to bf16. The roofline is HBM: 288 bytes read and
    1024 written per entry, plus the positions."""
    import numpy as np
    import torch

    import synth
    from top_fp4_lightning_amd import pipeline

    nseq, n, k, nsel, seed = 64, 1 << 20, 512, 5, 12
    t = time.perf_counter()
    sels = [synth.selections(seed + i, nseq, n, k) for i in range(nsel)]
    plan = pipeline.MainKVGather(nseq, n, sels, lambda b, p: synth.mkv_rows_of(seed, b, p))
    torch.cuda.synchronize()
    log(f"kv_gather_1m: {nseq} x {n} main-KV entries ({plan.codes.numel() + plan.scales.numel()} bytes), "
        f"{plan.rows_written} rows written; setup {time.perf_counter() - t:.1f} s")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for i in range(nsel):
            plan.gather(i)
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsel)]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        for i in range(nsel):
            evs[st][i][0].record(stream)
            plan.gather(i)
            evs[st][i][1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b) for row in evs for a, b in row]))
    entries = nseq * k * nsel
    per_launch = nseq * k * (288 + 1024 + 4) + nseq * (8 + 4)
    achieved = per_launch / (launch_ms / 1000.0) / 1e9
    res = {
        "metric": "main-KV entries gathered and dequantised to bf16 per s; % of HBM roofline",
        "value": entries / (ms_step / 1000.0), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e2m1+e4m3 -> bf16", "data": "synthetic (seeded RMS-normalised bf16 rows)",
        "config": {"workload": "kv_gather_1m: 64 x 1048576 FP4 main-KV entries, 5 selections of 512 per query "
                               "per step (Full + 4 Reindex layers)", "batch": nseq, "context": n, "k": k,
                   "selections": nsel},
        "gather_ms": launch_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "gather_kv_kernel",
                     "algorithmic_bytes_per_launch": per_launch},
    }
    if not args.no_cpu_baseline:
        import oracle

        nq_s = 16
        rows = [synth.mkv_rows_of(seed, np.full(k, b), sels[0][b]) for b in range(nq_s)]
        qc, qs = oracle.mkv_quantize(np.concatenate(rows))
        base = np.arange(nq_s, dtype=np.int64) * k
        idx = np.tile(np.arange(k, dtype=np.int32), (nq_s, 1))
        t1 = time.perf_counter()
        oracle.mkv_gather(qc, qs, base, np.full(nq_s, k, dtype=np.int64), idx)
        dt = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": nq_s * k / dt, "unit": "entries/s", "cores": 1, "kind": "oracle",
                               "sample": f"gather-dequantise of {nq_s} queries x {k} entries (one selection); "
                                         f"{dt:.2f} s on 1 thread", "seconds": round(dt, 3)}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fullscan_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: time replays of the step captured in a HIP graph")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 512 MiB device-to-device 5 times (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the indexer shards by "
              "sequence with no exchange, or by key range with one all-gather of per-shard candidates)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import top_fp4_lightning_amd as fx
    from top_fp4_lightning_amd import pipeline

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel(), "launches": 5}), flush=True)
        return 0
    if args.workload == "kv_gather_1m":
        return bench_kv_gather(args)
    if args.workload == "token_1m":
        return bench_token(args)
    if args.workload == "mask_form_1m":
        return bench_mask_form(args)
    wl = synth.config(args.workload)
    if args.workload == "prefill_128k":
        return bench_prefill(wl, args)
    return bench_decode(wl, args)

if __name__ == "__main__":
    sys.exit(main())
