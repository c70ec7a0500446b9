"""Pins for the oracle's top-k, block maxima, pin and candidate pool (CPU only).

Brute force on tiny inputs (repeated argmax), the pool's defining properties, the short-context
rule, the nesting invariant top-k in pool in visible, and gather form = mask form for Reindex.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth


def brute_topk(I, k):
    I = list(I)
    out = []
    alive = [np.isfinite(v) or v == np.inf for v in I]
    for _ in range(k):
        best = -1
        for s, v in enumerate(I):
            if alive[s] and (best < 0 or v > I[best]):
                best = s  # strict '>' keeps the lower index on ties
        if best < 0:
            break
        out.append(best)
        alive[best] = False
    return out + [-1] * (k - len(out))


def brute_pool(bm, n, block, keep):
    nb = (n + block - 1) // block
    vals = [np.inf if b == (n - 1) // block else bm[b] for b in range(nb)]
    chosen = brute_topk(vals, min(keep, nb))
    return sorted(b for b in chosen if b >= 0 and vals[b] > -np.inf)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(-4, 4), min_size=0, max_size=40), st.integers(1, 12))
def test_topk_bruteforce_with_ties(vals, k):
    I = np.array(vals, dtype=np.float64)
    assert list(oracle.topk(I, k)) == brute_topk(I, k)


def test_topk_ignores_minus_inf_and_pads():
    I = np.array([1.0, -np.inf, 3.0, -np.inf, 2.0])
    assert list(oracle.topk(I, 5)) == [2, 4, 0, -1, -1]


@pytest.mark.parametrize("n", [1, 7, 8, 9, 15, 16, 17, 100])
def test_block_max_pads_last_block(n):
    rng = np.random.default_rng(n)
    I = rng.standard_normal(n)
    bm = oracle.block_max(I, 8)
    assert len(bm) == (n + 7) // 8
    for b in range(len(bm)):
        assert bm[b] == I[8 * b:min(8 * b + 8, n)].max()


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 60), st.integers(1, 6), st.integers(1, 9), st.integers(0, 2 ** 31))
def test_pool_bruteforce_scaled_down(n, block, keep, seed):
    rng = np.random.default_rng(seed)
    I = rng.integers(-3, 4, n).astype(np.float64)  # many ties
    bm = oracle.block_max(I, block)
    got = list(oracle.pool(bm, n, block, keep))
    assert got == brute_pool(bm, n, block, keep)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 511, 512, 513, 16383, 16384, 16385, 16392, 50000, 1 << 20])
def test_pool_definition_edges(n):
    rng = np.random.default_rng(n + 5)
    I = rng.standard_normal(n)
    bm = oracle.block_max(I, 8)
    pool = oracle.pool(bm, n, 8, 2048)
    nb = (n + 7) // 8
    assert len(pool) == min(2048, nb)
    assert np.all(np.diff(pool) > 0)
    if n == 0:
        return
    last = (n - 1) // 8
    assert last in set(pool.tolist())  # the newest block is always kept
    if nb <= 2048:  # short context: the pool is every visible position
        assert np.array_equal(pool, np.arange(nb))
    else:
        kept = np.zeros(nb, bool)
        kept[pool] = True
        kept_vals = np.where(np.arange(nb) == last, np.inf, bm)[kept]
        dropped = bm[~kept]
        assert kept_vals.min() >= dropped.max()


def test_topk_edges():
    for n in [0, 1, 511, 512, 513, 4096]:
        rng = np.random.default_rng(n)
        I = rng.standard_normal(n)
        t = oracle.topk(I, 512)
        cnt = min(n, 512)
        assert (t[:cnt] >= 0).all() and (t[cnt:] == -1).all()
        ref = np.lexsort((np.arange(n), -I))[:cnt]
        assert np.array_equal(t[:cnt], ref)


def decode_case(seed, n, layers=2):
    w = synth.decode_workload("t", seed, [n], layers=layers)
    s = w.signs()
    kc, ks = oracle.quantize(w.keys(0), s)
    q = [oracle.quantize(w.q(l, [0])[0], s) for l in range(layers + 1)]
    ws = [w.w(l, [0])[0] for l in range(layers + 1)]
    return w, kc, ks, q, ws


@pytest.mark.parametrize("n,block,keep,k", [(3000, 8, 64, 512), (3000, 8, 64, 63), (20000, 8, 2048, 512),
                                           (777, 4, 6, 5), (777, 4, 6, 8)])
def test_nesting_and_gather_equals_mask(n, block, keep, k):
    w, kc, ks, q, ws = decode_case(31 + n, n)
    I, _ = oracle.score_rows(q[0][0], q[0][1], ws[0], kc, ks)
    top = oracle.topk(I, k)
    pool = oracle.pool(oracle.block_max(I, block), n, block, keep)
    pos = set()
    for b in pool:
        pos.update(range(b * block, min(b * block + block, n)))
    assert pos <= set(range(n))
    if keep >= k + 1:
        # a top-k entry's block is outranked by at most k-1 unpinned blocks, so it is kept
        assert set(top[top >= 0].tolist()) <= pos
    for l in (1, 2):
        Il, _ = oracle.score_rows(q[l][0], q[l][1], ws[l], kc, ks)
        m = oracle.reindex_mask(Il, pool, block, k)
        g = oracle.reindex_gather(q[l][0], q[l][1], ws[l], kc, ks, pool, block, k)
        assert np.array_equal(m, g)
        assert set(m[m >= 0].tolist()) <= pos


def test_decode_batch_matches_pieces():
    n = [1500, 40, 17000]
    w = synth.decode_workload("t", 41, n, layers=2)
    s = w.signs()
    kc, ks = oracle.quantize(np.concatenate([w.keys(b) for b in range(3)]), s)
    qc, qs = oracle.quantize(w.q(0), s)
    rq = [oracle.quantize(w.q(l), s) for l in (1, 2)]
    top, pools, rtop = oracle.decode_batch(kc, ks, w.k_base, w.n_vis, qc, qs, w.w(0),
                                           np.stack([r[0] for r in rq]), np.stack([r[1] for r in rq]),
                                           np.stack([w.w(l) for l in (1, 2)]), nthreads=3)
    for t in range(3):
        b0, nn = int(w.k_base[t]), int(w.n_vis[t])
        I, _ = oracle.score_rows(qc[t], qs[t], w.w(0)[t], kc[b0:b0 + nn], ks[b0:b0 + nn])
        assert np.array_equal(top[t], oracle.topk(I, 512))
        pool = oracle.pool(oracle.block_max(I), nn)
        assert np.array_equal(pools[t], pool)
        for li in range(2):
            Il, _ = oracle.score_rows(rq[li][0][t], rq[li][1][t], w.w(li + 1)[t], kc[b0:b0 + nn], ks[b0:b0 + nn])
            assert np.array_equal(rtop[li, t], oracle.reindex_mask(Il, pool))


@pytest.mark.parametrize("n,count", [(1, 1), (100, 5), (1000, 125), (4097, 300)])
def test_mask_pool_keeps_exactly_the_pooled_positions(n, count):
    rng = np.random.default_rng(n + count)
    I = rng.standard_normal(n)
    nb = (n + 7) // 8
    pool = rng.permutation(nb)[:min(count, nb)].astype(np.int32)
    m = oracle.mask_pool(I, pool)
    blocks = np.arange(n) // 8
    inside = np.isin(blocks, pool)
    assert np.array_equal(m[inside], I[inside]) and np.isneginf(m[~inside]).all()
    assert inside.sum() == sum(min(8, n - 8 * int(b)) for b in pool)
    # the official form: a boolean table per query; masking and top-k equals the mask-form Reindex
    assert np.array_equal(oracle.topk(m, 7), oracle.reindex_mask(I, pool, 8, 7))
