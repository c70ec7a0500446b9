"""Full-size GPU runs of every workload, checked against the oracle.

The GPU path runs exactly as the benchmark runs it (DecodePlan / PrefillPlan over the whole
batch). Every query is checked element by element on a seeded sample: the block maxima of about
256 of its blocks (and of its last, ragged block) and, for decode, the gathered scores of 64 of
its pooled slots in every layer, against the oracle's scores of those keys (quantised by the
oracle from the seeded generator, never from GPU output). For a few sampled queries the oracle
also scores every visible key; the GPU's top-512, pool and Reindex selections of those queries
must match it under the boundary tolerance. The oracle calls are spread over host threads
(ctypes releases the GIL).
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


class KeyBlocks:
    """bf16 key rows of whole 8-position blocks of one sequence, regenerated from the seeded
    generator (the planted set and shift computed once per sequence)."""

    def __init__(self, wl, b):
        self.wl, self.b = wl, b
        self.n = int(wl.seq_len[b])
        self.pos = wl.planted(b)
        self.shift = synth.plant_shift(wl.q(0, [int(wl.plant_query[b])])[0]) if len(self.pos) else None

    def rows(self, start, cnt):
        rows = synth.normal_bf16(self.wl.seed, synth.TAG_K, self.b, start * 128, cnt * 128).reshape(cnt, 128)
        if self.shift is not None:
            synth.lib().synth_apply_plant(rows.ctypes.data, start, cnt, self.pos.ctypes.data, len(self.pos),
                                          self.shift.ctypes.data)
        return rows


def sample_blocks(rng, nb, count=256):
    """about `count` distinct seeded block ids of a row of nb blocks, always with the last one"""
    if nb <= 0:
        return np.zeros(0, np.int64)
    pick = rng.choice(nb, size=min(count, nb), replace=False)
    return np.unique(np.concatenate([pick, [nb - 1]])).astype(np.int64)


def check_sampled_block_maxima(wl, t, n, bm_gpu_row, kb: "KeyBlocks", qc, qs, w, rng, count=256, what=""):
    """GPU block maxima of query t on sampled blocks, against the oracle's scores of their keys"""
    nb = (n + 7) // 8
    blocks = sample_blocks(rng, nb, count)
    rows, owner = [], []
    for blk in blocks:
        s0 = 8 * int(blk)
        cnt = min(8, n - s0)
        rows.append(kb.rows(s0, cnt))
        owner.extend([int(blk)] * cnt)
    rows = np.concatenate(rows) if rows else np.zeros((0, 128), np.uint16)
    kc, ks = oracle.quantize(rows, wl.signs(), nthreads=1)
    I, A = oracle.score_rows(qc, qs, w, kc, ks)
    owner = np.asarray(owner)
    for blk in blocks:
        m = owner == blk
        ref, a = I[m].max(), A[m].max()
        got = float(bm_gpu_row[blk])
        assert abs(got - ref) <= 1e-5 * max(a, 1e-30), f"{what} q{t} block {blk}: {got!r} vs {ref!r}"
    return len(blocks)


def check_sampled_pool_scores(wl, t, n, layer, pool_row, cnt, scores_row, kb, signs, rng, count=64, what=""):
    """gathered pool-order scores of one layer on sampled slots, against the oracle"""
    slots = np.arange(8 * int(cnt))
    if len(slots) == 0:
        return 0
    pick = np.sort(rng.choice(slots, size=min(count, len(slots)), replace=False))
    pos = 8 * pool_row[pick // 8].astype(np.int64) + pick % 8
    valid = pos < n
    for s_, p_ in zip(pick[~valid], pos[~valid]):
        assert np.isneginf(scores_row[s_]), f"{what} q{t} layer {layer} slot {s_} past n"
    pick, pos = pick[valid], pos[valid]
    if len(pos) == 0:
        return 0
    rows = np.concatenate([kb.rows(int(p_), 1) for p_ in pos])
    kc, ks = oracle.quantize(rows, signs, nthreads=1)
    qc, qs = oracle.quantize(wl.q(layer, [t])[0], signs)
    I, A = oracle.score_rows(qc, qs, wl.w(layer, [t])[0], kc, ks)
    got = scores_row[pick].astype(np.float64)
    bad = np.abs(got - I) > 1e-5 * np.maximum(A, 1e-30)
    assert not bad.any(), f"{what} q{t} layer {layer}: {int(bad.sum())} gathered scores out of tolerance"
    return len(pos)


def check_every_decode_query(wl, out, what):
    """element-wise coverage of every query of a decode batch: sampled block maxima of the Full
    scan and sampled gathered scores of every layer"""
    plan = out["plan"]
    signs = wl.signs()
    bm_gpu = out["block_max"].cpu().numpy()
    pbk, pcn = out["pool_blocks"].cpu().numpy(), out["pool_count"].cpu().numpy()
    ps = [x.cpu().numpy() for x in plan.pool_scores]
    seqs = {}

    def one(t):
        rng = np.random.default_rng(1000 + t)
        b = int(wl.qseq[t])
        n = int(wl.n_vis[t])
        kb = seqs[b]
        qc, qs = oracle.quantize(wl.q(0, [t])[0], signs)
        nblk = check_sampled_block_maxima(wl, t, n, bm_gpu[t], kb, qc, qs, wl.w(0, [t])[0], rng, what=what)
        nsl = 0
        for layer in range(plan.layers + 1):
            nsl += check_sampled_pool_scores(wl, t, n, layer, pbk[t], pcn[t], ps[layer][t], kb, signs, rng, what=what)
        return nblk, nsl

    for b in sorted(set(int(x) for x in wl.qseq)):
        seqs[b] = KeyBlocks(wl, b)
    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(one, range(wl.nq)))
    print(f"{what}: every query checked: {sum(r[0] for r in res)} sampled block maxima, "
          f"{sum(r[1] for r in res)} sampled gathered scores", flush=True)


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
    check_every_decode_query(wl, out, "fullscan_1m")
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
    check_every_decode_query(wl, out, "fullscan_512k")
    check_decode_queries(wl, out, sample=[3])


def test_decode_batch64(pl):
    # 64 sequences with lengths in [64K, 128K]
    wl = synth.config("decode_batch64")
    out = run_decode(pl, wl)
    check_every_decode_query(wl, out, "decode_batch64")
    order = np.argsort(wl.n_vis)
    check_decode_queries(wl, out, sample=[int(order[0]), int(order[-1]), 17])


def test_reindex_1m(pl):
    # 64 x 2^20 keys, pool from the Full layer, 4 Reindex layers with their own q and w
    wl = synth.config("reindex_1m")
    out = run_decode(pl, wl)
    check_every_decode_query(wl, out, "reindex_1m")
    check_decode_queries(wl, out, sample=[0, 63])


def test_spec_decode_1m(pl):
    # 8 x 2^20 keys, 6 positions per sequence (the token + 5 draft positions) scanned together by
    # the many-query kernel; pool, Full top-512 and 4 Reindex layers per position
    wl = synth.config("spec_decode_1m")
    out = run_decode(pl, wl)
    check_every_decode_query(wl, out, "spec_decode_1m")
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
    bm_gpu = plan.block_max.cpu().numpy()

    def every(t):
        # every query: its block maxima on ~256 seeded blocks (and its last, ragged one)
        rng = np.random.default_rng(5000 + t)
        n = int(wl.n_vis[t])
        nb = (n + 7) // 8
        blocks = sample_blocks(rng, nb, 256)
        pos = (8 * blocks[:, None] + np.arange(8)[None, :]).reshape(-1)
        pos = pos[pos < n]
        qc, qs = oracle.quantize(wl.q(0, [t])[0], s)
        I, A = oracle.score_rows(qc, qs, wl.w(0, [t])[0], kc[pos], ks[pos])
        owner = pos // 8
        for blk in blocks:
            m = owner == blk
            ref, a = I[m].max(), A[m].max()
            assert abs(float(bm_gpu[t, blk]) - ref) <= 1e-5 * max(a, 1e-30), f"prefill q{t} block {blk}"
        return len(blocks)

    with ThreadPoolExecutor(THREADS) as ex:
        nblk = sum(ex.map(every, range(wl.nq)))
    print(f"prefill_128k: every query checked: {nblk} sampled block maxima", flush=True)
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
