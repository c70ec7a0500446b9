#!/usr/bin/env python3
"""Benchmark: the FP4 lightning indexer's decode hot path at 1M context on one MI355X.

Headline workload ("fullscan_1m"): 8 sequences x 2^20 visible compressed keys (decoder, m = 1),
one query each, 32 heads x 128 dims, MXFP4 queries and keys, synthetic seeded inputs. One step is
the whole hot path for that batch: quantise the Full layer's queries, scan every key (block-8
maxima fused), build the candidate pool (pin + top-2048 blocks), take the Full layer's top-512,
then 4 Reindex layers (quantise their queries, gather-score the pool, top-512 each).

Prints one JSON line: entries scored per second over the step (Full-layer keys + pooled keys of
the Reindex layers), top-512 queries per second, the scan kernel's HBM roofline fraction
(achieved from HIP events around the scan launches of the timed steps), the same step cold (1 GiB
written before each repetition, outside its events) and the pool gather cold and warm, a record
for each other configuration of the problem statement (configs: decode_32k, decode_batch64,
reindex_1m, fullscan_512k, prefill_128k, each warm and cold with the roofline of its dominant
kernel), and the CPU oracle timed on all host cores on the step's work.
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


def host_threads() -> int:
    """threads for the CPU baseline: every core the process may use (the machine's CPU share, as
    OMP_NUM_THREADS states it when set)"""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, target_s: float = 5.0, runs: int = 3, chunk: int = 1 << 14) -> dict:
    """The oracle (plain C, as it stands) on all host cores, timed on the same work as the GPU
    step: the Full layer of every query (score all visible keys, top-512, block maxima, pin,
    top-2048 pool) and the Reindex layers (score the pooled keys with each layer's query,
    top-512). Threads take (query, key-chunk) units of the Full layer, then one query per unit
    for the selections and the Reindex layers. When the whole step would take longer than about
    `target_s` per run, each query's Full layer covers only its first 2^-m of its visible keys
    (halved until it fits); its cost is linear in that length. The Reindex layers' units run
    side by side (their queries are all present in the synthetic workload). The oracle quantises the
    keys first (untimed setup, as the GPU's key cache is); the queries are quantised inside the
    timed region, as on the GPU. Median of `runs` runs."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    threads = host_threads()
    s = wl.signs()
    nq, layers = wl.nq, wl.layers
    qraw = [wl.q(layer) for layer in range(layers + 1)]
    wraw = [wl.w(layer) for layer in range(layers + 1)]
    # calibration: one chunk of keys per thread, all threads at once (wall time per key scored)
    kc0, ks0 = oracle.quantize(wl.keys(int(wl.qseq[0]), 0, chunk), s, nthreads=threads)
    qc0, qs0 = oracle.quantize(qraw[0][0], s)
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda _: oracle.score_rows(qc0, qs0, wraw[0][0], kc0, ks0), range(threads)))
        per_key = (time.perf_counter() - t0) / (chunk * threads) * threads
    full = int(max(wl.n_vis))
    keys_per_q = full
    def est(m):  # seconds of scoring per run on all threads
        nn = np.minimum(wl.n_vis, m).astype(np.float64)
        return float(nn.sum() + layers * np.minimum(nn, 8 * wl.topk_blocks).sum()) * per_key / threads

    while keys_per_q > chunk and est(keys_per_q) > target_s:
        keys_per_q //= 2
    n = np.minimum(wl.n_vis.astype(np.int64), keys_per_q)
    log(f"cpu baseline: {threads} threads, {per_key * 1e6:.1f} us per key per thread (all threads busy); Full layer over "
        f"{keys_per_q} keys per query; oracle quantises the keys (untimed)")
    kc, ks = {}, {}
    for b in sorted(set(int(x) for x in wl.qseq)):
        kc[b], ks[b] = oracle.quantize(wl.keys(b, 0, int(n[list(wl.qseq).index(b)])), s, nthreads=threads)

    def one_run():
        t_start = time.perf_counter()
        qz = [oracle.quantize(qraw[layer], s, nthreads=threads) for layer in range(layers + 1)]
        I = [np.empty(int(n[t])) for t in range(nq)]
        A = [np.empty(int(n[t])) for t in range(nq)]

        def full_unit(u):
            t, c0 = u
            b = int(wl.qseq[t])
            c1 = min(int(n[t]), c0 + chunk)
            I[t][c0:c1], A[t][c0:c1] = oracle.score_rows(qz[0][0][t], qz[0][1][t], wraw[0][t], kc[b][c0:c1],
                                                         ks[b][c0:c1])

        def select(t):
            top = oracle.topk(I[t], wl.k)
            pool = oracle.pool(oracle.block_max(I[t], 8), int(n[t]), 8, wl.topk_blocks)
            return top, pool

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(full_unit, [(t, c0) for t in range(nq) for c0 in range(0, int(n[t]), chunk)]))
            sel = list(ex.map(select, range(nq)))

            def reindex(u):
                layer, t = u
                b = int(wl.qseq[t])
                oracle.reindex_gather(qz[layer][0][t], qz[layer][1][t], wraw[layer][t], kc[b][:int(n[t])],
                                      ks[b][:int(n[t])], sel[t][1], 8, wl.k)
                return int(min(8 * len(sel[t][1]), int(n[t])))

            entries = int(n.sum()) + sum(ex.map(reindex, [(l, t) for l in range(1, layers + 1) for t in range(nq)]))
        return time.perf_counter() - t_start, entries

    res = [one_run() for _ in range(runs)]
    secs = sorted(r[0] for r in res)
    dt = secs[len(secs) // 2]
    entries = res[0][1]
    sub = "every visible key" if keys_per_q >= full else f"the first {keys_per_q} visible keys"
    return {"value": entries / dt, "unit": "entries/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"the step's work for all {nq} queries: Full layer over {sub} of each query (score, top-512, "
                      f"block max, pin, top-2048 pool), then {layers} Reindex layers scoring the pooled keys "
                      f"(top-512 each); {entries} entries scored per run; median of {runs} runs "
                      f"({', '.join(f'{x:.2f}' for x in secs)} s) on {threads} threads",
            "seconds": round(dt, 3), "entries_per_run": entries}


MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak, published
FLUSH_BYTES = 1 << 30


class Flusher:
    """Before each cold repetition, outside its event pair: writes 1 GiB of device memory with a
    plain fill kernel (a changing non-zero byte, so never a memset), then reads it back with a
    reduction. The 4 MB L2s and the 256 MB last-level cache then hold none of the workload's
    inputs, and the lines they do hold are clean, so the measured kernel's misses do not also pay
    for writing the flush's dirty lines back."""

    def __init__(self):
        import torch

        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.v = 0

    def __call__(self):
        import torch

        self.v = self.v % 250 + 1
        self.buf.fill_(self.v)
        self.buf.view(torch.int64).sum()


def host_ahead(steps: int = 1):
    """An untimed spin kernel before a warm timed region (about 0.3 ms plus 0.1 ms per step), so
    that the host has enqueued the timed launches before the GPU reaches them (small steps are
    otherwise bound by the host's launch rate rather than by the device)."""
    import torch

    torch.cuda._sleep(700_000 + 250_000 * max(0, steps))


def _pair():
    import torch

    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2] if xs else float("nan")


def hbm_roofline(bytes_per_launch: int, ms: float, kernel: str, traffic=None) -> dict:
    achieved = bytes_per_launch / (ms / 1000.0) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel,
            "algorithmic_bytes_per_launch": bytes_per_launch, "launch_ms": ms}


def mfma_roofline(flop: float, ms: float, kernel: str, traffic=None, bytes_per_launch=None) -> dict:
    achieved = flop / (ms / 1000.0) / 1e12
    r = {"bound": "mfma", "achieved": achieved, "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
         "frac": achieved / MFMA_FP4_PEAK_TFLOPS, "traffic": traffic, "kernel": kernel,
         "algorithmic_flop_per_launch": flop, "launch_ms": ms}
    if bytes_per_launch is not None:
        r["algorithmic_bytes_per_launch"] = bytes_per_launch
        r["hbm_achieved_gbs"] = bytes_per_launch / (ms / 1000.0) / 1e9
        r["hbm_frac"] = r["hbm_achieved_gbs"] / HBM_PEAK_GBS
    return r


def prefill_record(wl, reps: int, warmup: int, flush) -> dict:
    """Chunked prefill: 4096 consecutive queries on 131072 keys, causal; the step is quantise q,
    the many-query scan (block maxima), top-512 blocks per query, re-score of those 4096 keys,
    final top-512. The roofline is the scan's FP4 matrix throughput. Warm: steps back to back;
    cold: the caches flushed before each step."""
    import torch

    from top_fp4_lightning_amd import pipeline

    t = time.perf_counter()
    dev = pipeline.DeviceWorkload.from_workload(wl, group=wl.nq)
    torch.cuda.synchronize()
    log(f"workload {wl.name}: {wl.nq} queries, {wl.total_keys} keys; setup {time.perf_counter() - t:.1f} s")
    plan = pipeline.PrefillPlan(dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    scan_w = [_pair() for _ in range(reps)]
    whole = _pair()
    host_ahead()
    whole[0].record(stream)
    for i in range(reps):
        plan.run(events=scan_w[i])
    whole[1].record(stream)
    torch.cuda.synchronize()
    step_cold, scan_c = [_pair() for _ in range(reps)], [_pair() for _ in range(reps)]
    for i in range(reps):
        flush()
        step_cold[i][0].record(stream)
        plan.run(events=scan_c[i])
        step_cold[i][1].record(stream)
    torch.cuda.synchronize()
    ms_warm = whole[0].elapsed_time(whole[1]) / reps
    ms_cold = _median(_ms(step_cold))
    scan_warm, scan_cold = sum(_ms(scan_w)) / reps, _median(_ms(scan_c))
    pairs = int(wl.n_vis.sum())
    flop = 2.0 * 4096.0 * pairs
    sb = int(wl.total_keys) * 68 + wl.nq * (32 * 68 + 32 * 4) + int(sum((n + 7) // 8 for n in wl.n_vis)) * 4
    rec = {"workload": "prefill_128k: 4096 queries x 131072 keys, causal (query i sees <= 126976+i)",
           "metric": "(query, key) pairs scored/s, top-512 queries/s; % of FP4 MFMA roofline",
           "reps": reps, "ms_per_step": ms_warm, "ms_per_step_cold": ms_cold,
           "pairs_per_s": pairs / (ms_warm / 1000.0), "pairs_per_s_cold": pairs / (ms_cold / 1000.0),
           "queries_per_s": wl.nq / (ms_warm / 1000.0), "scan_ms": scan_warm, "scan_ms_cold": scan_cold,
           "roofline": mfma_roofline(flop, scan_warm, "score_multi_kernel",
                                     measured_traffic("score_multi_prefill_128k_traffic"), sb),
           "roofline_cold": mfma_roofline(flop, scan_cold, "score_multi_kernel", None, sb)}
    del plan, dev
    torch.cuda.empty_cache()
    return rec


def bench_prefill(wl, args) -> int:
    rec = prefill_record(wl, args.steps, args.warmup, Flusher())
    print(json.dumps({
        "metric": "prefill (query, key) pairs scored/s; % of FP4 MFMA roofline",
        "value": rec["pairs_per_s"], "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": rec["workload"]}, **{k: v for k, v in rec.items() if k not in ("workload", "metric")},
    }), flush=True)
    return 0


DECODE_CONFIGS = {
    "fullscan_1m": "fullscan_1m decode step: batch 8 x 1048576 keys (m=1), Full scan + top-512 + "
                   "pool(2048 blocks of 8) + 4 Reindex layers",
    "fullscan_512k": "fullscan_512k decode step: batch 8 x 524288 keys (encoder shape, m=2), Full scan + "
                     "top-512 + pool(2048 blocks of 8)",
    "decode_32k": "decode_32k: 1 query x 32768 keys, Full scan + top-512 + pool(2048 of 4096 blocks)",
    "decode_batch64": "decode_batch64: 64 sequences x U[65536, 131072] keys, Full scan + top-512 + "
                      "pool(2048 blocks of 8)",
    "reindex_1m": "reindex_1m: 64 sequences x 1048576 keys, Full pass + pool(2048 blocks of 8) + 4 Reindex "
                  "layers gathering the 16384 pooled keys, top-512 each",
    "spec_decode_1m": "spec_decode_1m verify step: batch 8 x 1048576 keys (m=1), 6 positions per sequence "
                      "(token + 5 draft), Full scan + top-512 + pool(2048 blocks of 8) + 4 Reindex layers",
}


class DecodeStep:
    """One decode step through the plan (quantise, Full scan, pool, Full top-512 through the
    pool, then per Reindex layer quantise, gather, top-512), with optional HIP event pairs
    around the scan and around each gather launch (recorded on the launch stream)."""

    def __init__(self, wl):
        import torch

        from top_fp4_lightning_amd import pipeline

        t = time.perf_counter()
        self.wl = wl
        self.dev = pipeline.DeviceWorkload.from_workload(wl)
        torch.cuda.synchronize()
        log(f"workload {wl.name}: {wl.nq} queries, {wl.total_keys} keys, {wl.layers} Reindex layers; "
            f"setup {time.perf_counter() - t:.1f} s")
        self.plan = pipeline.DecodePlan(self.dev)
        self.stream = torch.cuda.current_stream()
        # the timed steps replay the step's launches with their arguments marshalled once (the same
        # launches as self(), without the per-call host work that otherwise rivals the step itself)
        self.replay = self.plan.compiled(self.stream)
        import top_fp4_lightning_amd as fx

        with fx.record() as calls:
            for layer in range(self.plan.layers + 1):
                self.plan.pool_gather(layer, self.stream)
        self.gather_replay = fx.Recorded(calls)
        n_vis = [int(x) for x in wl.n_vis]
        self.n_vis = n_vis
        self.pool_pos = int(sum(min(n, 8 * min(2048, (n + 7) // 8)) for n in n_vis))
        self.entries = int(sum(n_vis)) + self.plan.layers * self.pool_pos
        self.queries = wl.nq * (1 + self.plan.layers)
        self.slots = wl.nq * self.plan.max_blocks * 8
        # gather: 68 B per pooled key, q (32 x 68 B) + w (128 B) per query, 4 B per score slot written
        self.gather_bytes = self.pool_pos * 68 + wl.nq * (32 * 68 + 32 * 4) + self.slots * 4

    def __call__(self, scan_ev=None, gather_ev=None, flush=None):
        p = self.plan
        p.quantize(0)
        if scan_ev is not None:
            scan_ev[0].record(self.stream)
        p.full_scan()
        if scan_ev is not None:
            scan_ev[1].record(self.stream)
        p.build_pool()
        for layer in range(p.layers + 1):
            if layer:
                p.quantize(layer)
            if flush is not None:
                flush()
            p.pool_select(layer, events=None if gather_ev is None else gather_ev[layer])

    def scan_roofline(self, ms: float, traffic=None) -> dict:
        wl, dev = self.wl, self.dev
        if dev.group == 1:
            return hbm_roofline(scan_bytes(self.n_vis, wl.nq), ms, "score_full_kernel", traffic)
        flop = 2.0 * 4096.0 * float(sum(self.n_vis))
        groups = [self.n_vis[i:i + dev.group] for i in range(0, len(self.n_vis), dev.group)]
        sb = (sum(max(g) * 68 for g in groups) + wl.nq * (32 * 68 + 32 * 4) +
              sum((n + 7) // 8 for n in self.n_vis) * 4)
        return mfma_roofline(flop, ms, "score_multi_kernel", traffic, sb)

    def measure(self, reps: int, warmup: int, flush) -> dict:
        """warm (steps back to back) and cold (caches flushed before each step) step times, the
        scan's launch time in both, and the pool gather per layer: cold (caches flushed right
        before the gather launch) and warm (gathers launched back to back)"""
        import torch

        p, L = self.plan, self.plan.layers
        for _ in range(warmup):
            self()
        torch.cuda.synchronize()
        # whole steps with no event inside them (an event pair between launches costs a few us);
        # the scan's own time in separate passes of the same steps
        whole = _pair()
        host_ahead(reps)
        whole[0].record(self.stream)
        for i in range(reps):
            self.replay()
        whole[1].record(self.stream)
        torch.cuda.synchronize()
        scan_w = [_pair() for _ in range(reps)]
        host_ahead(reps)
        for i in range(reps):
            self(scan_ev=scan_w[i])
        torch.cuda.synchronize()
        step_c, scan_c = [_pair() for _ in range(reps)], [_pair() for _ in range(reps)]
        for i in range(reps):
            flush()
            step_c[i][0].record(self.stream)
            self.replay()
            step_c[i][1].record(self.stream)
        torch.cuda.synchronize()
        for i in range(reps):
            flush()
            self(scan_ev=scan_c[i])
        torch.cuda.synchronize()
        g_cold = [[_pair() for _ in range(L + 1)] for _ in range(reps)]
        for i in range(reps):
            self(gather_ev=g_cold[i], flush=flush)
        g_warm = _pair()
        host_ahead(reps)
        g_warm[0].record(self.stream)
        for _ in range(reps):
            self.gather_replay()
        g_warm[1].record(self.stream)
        torch.cuda.synchronize()
        ms_warm = whole[0].elapsed_time(whole[1]) / reps
        ms_cold = _median(_ms(step_c))
        scan_warm, scan_cold = sum(_ms(scan_w)) / reps, _median(_ms(scan_c))
        gc = _median([x for row in g_cold for x in _ms(row)])
        gw = g_warm[0].elapsed_time(g_warm[1]) / (reps * (L + 1))
        gb = self.gather_bytes
        return {"reps": reps, "ms_per_step": ms_warm, "ms_per_step_cold": ms_cold,
                "entries_per_s": self.entries / (ms_warm / 1000.0),
                "entries_per_s_cold": self.entries / (ms_cold / 1000.0),
                "top512_queries_per_s": self.queries / (ms_warm / 1000.0),
                "top512_queries_per_s_cold": self.queries / (ms_cold / 1000.0),
                "full_scan_entries_per_s": sum(self.n_vis) / (scan_warm / 1000.0),
                "scan_ms": scan_warm, "scan_ms_cold": scan_cold,
                "gather": {"kernel": "score_gather_kernel", "algorithmic_bytes_per_launch": gb,
                           "ms_cold": gc, "frac_cold": gb / (gc / 1000.0) / 1e9 / HBM_PEAK_GBS,
                           "ms_warm": gw, "frac_warm": gb / (gw / 1000.0) / 1e9 / HBM_PEAK_GBS,
                           "cold_protocol": "1 GiB written and read back right before each gather launch, one event pair "
                                            "per launch",
                           "warm_protocol": "every layer's gather launched back to back between one event pair"}}


def decode_record(name: str, reps: int, warmup: int, flush) -> dict:
    import torch

    import synth

    wl = synth.config(name)
    st = DecodeStep(wl)
    m = st.measure(reps, warmup, flush)
    traffic = measured_traffic("score_full_fullscan_1m_traffic") if name == "fullscan_1m" else None
    rec = {"workload": DECODE_CONFIGS.get(name, name), **m,
           "roofline": st.scan_roofline(m["scan_ms"], traffic), "roofline_cold": st.scan_roofline(m["scan_ms_cold"])}
    if name == "reindex_1m":
        # the Reindex layers' gather is this workload's headline kernel (HBM on gathered bytes)
        g = m["gather"]
        rec["gather"]["traffic"] = measured_traffic("score_gather_reindex_1m_traffic")
        rec["roofline_gather_cold"] = hbm_roofline(st.gather_bytes, g["ms_cold"], "score_gather_kernel",
                                                   rec["gather"]["traffic"])
        rec["roofline_gather_warm"] = hbm_roofline(st.gather_bytes, g["ms_warm"], "score_gather_kernel",
                                                   rec["gather"]["traffic"])
        rec["reindex_queries_per_s"] = wl.nq * wl.layers / (m["ms_per_step"] / 1000.0)
    del st
    torch.cuda.empty_cache()
    return rec


def bench_decode(wl, args) -> int:
    """One decode step per timed iteration (quantise, Full scan, pool, Full top-512 through the
    pool, Reindex layers). With one query per sequence the Full scan is the single-query kernel
    and the roofline is HBM; with several positions per sequence (speculative verification) it is
    the many-query kernel and the roofline is FP4 MFMA.

    The timed region follows the bench contract: `warmup` untimed steps, then exactly `steps`
    steps back to back between two synchronisations (the wall clock gives ms_per_step). The steps
    are the plan's launches with their arguments marshalled once (DecodePlan.compiled): the
    per-call Python work of the binding costs the host about as long as the device needs for a
    step, and would otherwise be what the clock measures (ms_per_step_eager reports that path).
    HIP events on the launch stream around each scan launch, in separate passes, give the scan's
    roofline. Afterwards, outside that region, the same plan is measured warm and cold
    (DecodeStep.measure), and in the default run every other configuration gets its own record
    (configs)."""
    import torch

    st = DecodeStep(wl)
    plan = st.plan
    for _ in range(args.warmup):
        st.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / args.steps
    # the same steps through the binding's per-call marshalling, for comparison
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1000.0 / args.steps
    if args.graph:
        # the whole step captured once in a HIP graph (the plan allocates nothing and the library
        # issues no memsets) and replayed: no per-launch host work inside the timed region
        side = torch.cuda.Stream()
        side.wait_stream(st.stream)
        with torch.cuda.stream(side):
            plan.run(stream=side)
        st.stream.wait_stream(side)
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
    flush = Flusher()
    extra = st.measure(min(args.steps, 20), 1, flush)
    scan_ms = extra["scan_ms"]
    traffic = measured_traffic("score_full_fullscan_1m_traffic") if wl.name == "fullscan_1m" else None
    res = {
        "metric": "indexer entries scored/s + top-512 queries/s at 1M ctx; % of HBM roofline",
        "value": st.entries / (ms_step / 1000.0),
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
                   "batch": wl.nseq, "positions_per_sequence": st.dev.group, "context": int(wl.seq_len[0]),
                   "reindex_layers": plan.layers, "k": 512, "pool_blocks": 2048, "block": 8},
        "top512_queries_per_s": st.queries / (ms_step / 1000.0),
        "full_scan_entries_per_s": int(sum(st.n_vis)) / (scan_ms / 1000.0),
        "scan_ms": scan_ms,
        "step_launch": "hip graph replay" if args.graph else "eager launches, arguments marshalled once",
        "ms_per_step_eager": ms_eager,
        "roofline": st.scan_roofline(scan_ms, traffic),
        "cold": {"protocol": "1 GiB written and read back before each repetition, outside its event pair",
                 "ms_per_step": extra["ms_per_step_cold"], "entries_per_s": extra["entries_per_s_cold"],
                 "scan_ms": extra["scan_ms_cold"], "roofline": st.scan_roofline(extra["scan_ms_cold"])},
        "gather": extra["gather"],
    }
    del st, plan
    torch.cuda.empty_cache()
    if args.all_configs:
        import synth

        configs = {}
        for name in ("decode_32k", "decode_batch64", "reindex_1m", "fullscan_512k"):
            configs[name] = decode_record(name, args.config_reps, 2, flush)
        configs["prefill_128k"] = prefill_record(synth.config("prefill_128k"), args.config_reps, 2, flush)
        res["configs"] = configs
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)
    return 0


def bench_select_ties(args) -> int:
    """Selection on rows of tied values (a zero query scores every key 0): the decode top-512 shape
    (8 rows of 16384 pool-order scores, k = 512) and the pool shape (8 rows of 131072 block maxima
    of 2^20 positions, top-2048 with the pin), each on seeded normal rows, rows of one value and
    rows of 97 distinct values, timed with HIP events per launch (median over the steps)."""
    import numpy as np
    import torch

    import top_fp4_lightning_amd as fx

    rng = np.random.default_rng(7)
    stream = torch.cuda.current_stream()

    def rows(kind, nq, n):
        if kind == "normal":
            return torch.from_numpy(rng.standard_normal((nq, n)).astype(np.float32)).cuda()
        if kind == "equal":
            return torch.zeros(nq, n, dtype=torch.float32, device="cuda")
        return torch.from_numpy(rng.integers(0, 97, (nq, n)).astype(np.float32)).cuda()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        evs = [_pair() for _ in range(args.steps)]
        for e in evs:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return _median(_ms(evs)) * 1000.0

    res = {"metric": "selection time on tied rows, us per launch (median)", "steps": args.steps,
           "warmup": args.warmup}
    nq, n, k = 8, 16384, 512
    ws = fx.workspace(fx.IDX_OP_TOPK, nq, n, k)
    out = torch.empty(nq, k, dtype=torch.int32, device="cuda")
    for kind in ("normal", "equal", "distinct97"):
        v = rows(kind, nq, n)
        res[f"topk_8x16384_k512_{kind}_us"] = timed(lambda: fx.idx_topk(v, n, k, out, ws))
    npos = 1 << 20
    nb = npos // 8
    ws = fx.workspace(fx.IDX_OP_BUILD_POOL, nq, npos, 2048)
    pb = torch.empty(nq, 2048, dtype=torch.int32, device="cuda")
    pc = torch.empty(nq, dtype=torch.int32, device="cuda")
    nv = torch.full((nq,), npos, dtype=torch.int32, device="cuda")
    for kind in ("normal", "equal", "distinct97"):
        v = rows(kind, nq, nb)
        res[f"pool_8x131072_k2048_{kind}_us"] = timed(lambda: fx.idx_build_pool(v, nv, npos, pb, pc, ws))
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
    replay = plan.compiled()  # the token's launches with their arguments marshalled once
    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / args.steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan.run()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1000.0 / args.steps
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
        "step_launch": "eager launches, arguments marshalled once", "ms_per_step_eager": ms_eager,
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
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="fullscan_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config-reps", type=int, default=10,
                    help="repetitions of each other configuration's record (warm and cold)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the records of the other configurations")
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
    if args.workload == "select_ties":
        return bench_select_ties(args)
    wl = synth.config(args.workload)
    if args.workload == "prefill_128k":
        return bench_prefill(wl, args)
    args.all_configs = args.workload == "fullscan_1m" and not args.headline_only
    return bench_decode(wl, args)

if __name__ == "__main__":
    sys.exit(main())
