"""Full-size GPU runs of every workload, checked against the oracle on sampled queries.

The GPU path runs exactly as the benchmark runs it (DecodePlan / PrefillPlan over the whole
batch). For a few sampled queries the oracle quantises that sequence's keys itself (from the
seeded generator, never from GPU output) and scores every visible key exactly; the GPU's top-512,
pool and Reindex selections of those queries must match it under the boundary tolerance.
The oracle calls are spread over host threads (ctypes releases the GIL).
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_pool_set, assert_topk_set, block_A

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
CHUNK = 1 << 16


@pytest.fixture(scope="module")
def pl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_fp4_lightning_amd import pipeline

    return pipeline


def oracle_keys(wl, b, n, signs):
    """the oracle's own quantisation of the first n keys of sequence b"""
    def part(s0):
        cnt = min(CHUNK, n - s0)
        return oracle.quantize(wl.keys(b, s0, cnt), signs, nthreads=1)

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(part, range(0, n, CHUNK)))
    if not parts:
        return np.zeros((0, 64), np.uint8), np.zeros((0, 4), np.uint8)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_scores(qc, qs, w, kc, ks):
    n = kc.shape[0]

    def part(s0):
        return oracle.score_rows(qc, qs, w, kc[s0:s0 + CHUNK], ks[s0:s0 + CHUNK])

    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(part, range(0, n, CHUNK)))
    if not parts:
        return np.zeros(0), np.zeros(0)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def check_decode_queries(wl, out, sample, k=512):
    s = wl.signs()
    top = out["topk"].cpu().numpy()
    pbk, pcn = out["pool_blocks"].cpu().numpy(), out["pool_count"].cpu().numpy()
    rtop = [r.cpu().numpy() for r in out["reindex_topk"]]
    bm_gpu = out["block_max"].cpu().numpy()
    for t in sample:
        b = int(wl.qseq[t])
        n = int(wl.n_vis[t])
        kc, ks = oracle_keys(wl, b, n, s)
        qc, qs = oracle.quantize(wl.q(0, [t])[0], s)
        I, A = oracle_scores(qc, qs, wl.w(0, [t])[0], kc, ks)
        assert_topk_set(top[t], I, A, k, f"{wl.name} full top-k q{t}")
        bm = oracle.block_max(I, 8)
        Ab = block_A(A, n)
        nb = (n + 7) // 8
        assert np.all(np.abs(bm_gpu[t, :nb] - bm) <= 1e-5 * np.maximum(Ab, 1e-30)), f"{wl.name} block max q{t}"
        gpool = pbk[t, :pcn[t]]
        assert_pool_set(gpool, bm, Ab, n, 2048, f"{wl.name} pool q{t}")
        pos = (8 * gpool[:, None].astype(np.int64) + np.arange(8)[None, :]).reshape(-1)
        pos = pos[pos < n]
        assert set(int(x) for x in top[t] if x >= 0) <= set(pos.tolist())
        for li in range(wl.layers):
            qc2, qs2 = oracle.quantize(wl.q(li + 1, [t])[0], s)
            kp, sp = kc[pos], ks[pos]
            I2p, A2p = oracle_scores(qc2, qs2, wl.w(li + 1, [t])[0], kp, sp)
            masked = np.full(n, -np.inf)
            masked[pos] = I2p
            A2 = np.zeros(n)
            A2[pos] = A2p
            assert_topk_set(rtop[li][t], masked, A2, k, f"{wl.name} reindex layer {li + 1} q{t}")


def run_decode(pl, wl):
    dev = pl.DeviceWorkload.from_workload(wl)
    plan = pl.DecodePlan(dev)
    out = pl.decode_step(dev, plan=plan)
    torch.cuda.synchronize()
    return out


def test_fullscan_1m(pl):
    # 8 x 2^20 keys (decoder, m = 1) with 4 Reindex layers: the benchmark's workload
    wl = synth.config("fullscan_1m")
    out = run_decode(pl, wl)
    check_decode_queries(wl, out, sample=[0, 7])


def test_mask_form_fullscan_1m(pl):
    # the training form at the benchmark's workload: every layer scores all 2^20 positions and
    # keeps the pooled ones (top-512 over the pooled positions, and the literal in-place mask with
    # a top-512 over whole rows); pools and every layer's top-512 equal the gather form's (whose
    # selections test_fullscan_1m pins to the oracle)
    wl = synth.config("fullscan_1m")
    dev = pl.DeviceWorkload.from_workload(wl)
    gather = pl.DecodePlan(dev).run()
    for write_mask in (False, True):
        mask = pl.MaskFormPlan(dev, write_mask=write_mask).run()
        torch.cuda.synchronize()
        assert torch.equal(mask.pool_count, gather.pool_count)
        assert torch.equal(mask.pool_blocks, gather.pool_blocks)
        for layer in range(mask.L):
            mi, mv = mask.layer_topk(layer)
            assert torch.equal(mi, gather.topk[layer]), f"layer {layer} write_mask={write_mask}"
            assert torch.equal(mv, gather.topk_val[layer]), f"layer {layer} write_mask={write_mask}"
        del mask


def test_fullscan_512k(pl):
    # 8 x 2^19 keys (encoder shape, m = 2)
    wl = synth.config("fullscan_512k")
    out = run_decode(pl, wl)
    check_decode_queries(wl, out, sample=[3])


def test_decode_batch64(pl):
    # 64 sequences with lengths in [64K, 128K]
    wl = synth.config("decode_batch64")
    out = run_decode(pl, wl)
    order = np.argsort(wl.n_vis)
    check_decode_queries(wl, out, sample=[int(order[0]), int(order[-1]), 17])


def test_reindex_1m(pl):
    # 64 x 2^20 keys, pool from the Full layer, 4 Reindex layers with their own q and w
    wl = synth.config("reindex_1m")
    out = run_decode(pl, wl)
    check_decode_queries(wl, out, sample=[0, 63])


def test_spec_decode_1m(pl):
    # 8 x 2^20 keys, 6 positions per sequence (the token + 5 draft positions) scanned together by
    # the many-query kernel; pool, Full top-512 and 4 Reindex layers per position
    wl = synth.config("spec_decode_1m")
    out = run_decode(pl, wl)
    check_decode_queries(wl, out, sample=[0, 5, 46])


def test_spec_decode_ragged(pl):
    # speculative verification over ragged sequences: a sequence of exactly 6 keys (its positions
    # see 1 .. 6), short ones, and one past 16384 blocks, so that every pool of the batch goes
    # through the long-row selection; every position checked
    wl = synth.spec_decode_workload("sps", 215, [6, 700, 20001, 140000], positions=6, layers=2)
    out = run_decode(pl, wl)
    check_decode_queries(wl, out, sample=list(range(wl.nq)))


def test_token_1m_encoder_layers(pl):
    # the per-token schedule: 3 encoder Full layers over their own 8 x 2^19 caches, then the
    # decoder step; sampled encoder queries against the oracle (the decoder part is
    # test_fullscan_1m's)
    encs, dec = synth.token_1m()
    plan = pl.TokenPlan([pl.DeviceWorkload.from_workload(w) for w in encs], pl.DeviceWorkload.from_workload(dec))
    plan.run()
    torch.cuda.synchronize()
    for wl, p, t in [(encs[0], plan.encoders[0], 2), (encs[2], plan.encoders[2], 6)]:
        out = {"topk": p.topk[0], "topk_val": p.topk_val[0], "pool_blocks": p.pool_blocks,
               "pool_count": p.pool_count, "block_max": p.block_max, "reindex_topk": []}
        check_decode_queries(wl, out, sample=[t])


def test_prefill_128k(pl):
    # 4096 queries on 131072 keys, query i sees positions <= 126976 + i
    wl = synth.config("prefill_128k")
    dev = pl.DeviceWorkload.from_workload(wl, group=wl.nq)
    plan = pl.PrefillPlan(dev).run()
    torch.cuda.synchronize()
    top = plan.topk.cpu().numpy()
    s = wl.signs()
    kc, ks = oracle_keys(wl, 0, int(wl.seq_len[0]), s)
    for t in [0, 1, 1000, 2047, 4094, 4095]:
        n = int(wl.n_vis[t])
        qc, qs = oracle.quantize(wl.q(0, [t])[0], s)
        I, A = oracle_scores(qc, qs, wl.w(0, [t])[0], kc[:n], ks[:n])
        assert_topk_set(top[t], I, A, 512, f"prefill q{t}")


def test_kv_gather_1m(pl):
    # 64 x 2^20 FP4 main-KV entries in HBM; one selection of 512 per query gathered to bf16;
    # sampled queries against the oracle's own quantisation and gather of the same rows
    nseq, n, k, seed = 64, 1 << 20, 512, 12
    sel = synth.selections(seed, nseq, n, k)
    plan = pl.MainKVGather(nseq, n, [sel], lambda b, p: synth.mkv_rows_of(seed, b, p))
    out = plan.gather(0)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in [0, 33, 63]:
        qc, qs = oracle.mkv_quantize(synth.mkv_rows_of(seed, np.full(k, b), sel[b]))
        want, bad = oracle.mkv_gather(qc, qs, np.zeros(1, np.int64), np.array([k], np.int64),
                                      np.arange(k, dtype=np.int32)[None, :])
        assert bad == 0 and np.array_equal(got[b], want[0]), f"query {b}"
