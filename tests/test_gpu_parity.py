"""GPU parity against the CPU oracle (needs an MI355X). Each call goes through the C ABI.

Bar: quantised codes and scales bit-exact; per-head dots bit-exact (whenever the oracle reports
them exactly representable, which the synthetic recipe always satisfies); scores within 1e-5 of
A = sum_j |w_j| ReLU(d_j); selections identical except entries within that tolerance of the k-th
value; selections over identical fp32 inputs identical.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (TOL, assert_pool_set, assert_scores_close, assert_topk_set, block_A, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_fp4_lightning_amd

    return top_fp4_lightning_amd


@pytest.fixture(scope="module")
def pl(fx):
    from top_fp4_lightning_amd import pipeline

    return pipeline


def bf16_rows(vals: np.ndarray) -> np.ndarray:
    return np.array([[synth.bf16_rne(float(v)) for v in row] for row in vals], dtype=np.uint16)


def special_rows():
    rows = []
    rows.append(np.zeros(128))
    r = np.random.default_rng(1).standard_normal(128); r[32:64] = 0.0; rows.append(r)  # one zero group
    rows.append(np.random.default_rng(2).standard_normal(128) * 2.0 ** -100)
    rows.append(np.random.default_rng(3).standard_normal(128) * 2.0 ** 90)
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6, 0.25] * 8)
    rows.append(g)
    rows.append(-np.abs(np.random.default_rng(4).standard_normal(128)))
    e = np.zeros(128); e[5] = 1.0; rows.append(e)
    e = np.zeros(128); e[100] = -3.0; e[3] = 1e-30; rows.append(e)
    return bf16_rows(np.array(rows))


@pytest.mark.parametrize("nrows", [1, 15, 16, 1000, 4133])
def test_quantize_bit_exact(fx, nrows):
    s = synth.signs(300 + nrows)
    x = synth.normal_bf16(300 + nrows, 3, 0, 0, nrows * 128).reshape(nrows, 128)
    x = np.concatenate([special_rows(), x])
    codes, scales = fx.idx_quantize_q(to_dev_bf16(x), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.quantize(x, s)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def run_full_scan(fx, pl, wl, want_dots=True):
    dev = pl.DeviceWorkload.from_workload(wl)
    nq, max_n = dev.nq, dev.max_n
    qc, qs = fx.idx_quantize_q(dev.q[0], dev.signs)
    scores = torch.full((nq, max_n), float("nan"), device="cuda")
    nb = (max_n + 7) // 8
    bm = torch.full((nq, nb), float("nan"), device="cuda")
    dots = torch.full((nq, 32, max_n), float("nan"), device="cuda") if want_dots else None
    fx.idx_score_full(dev.k_codes, dev.k_scales, dev.k_base, dev.n_vis, qc, qs, dev.w[0], max_n, scores=scores,
                      block_max=bm, head_dots=dots)
    torch.cuda.synchronize()
    return dev, scores.cpu().numpy(), bm.cpu().numpy(), (dots.cpu().numpy() if want_dots else None)


def test_score_full_parity(fx, pl):
    wl = synth.decode_workload("p", 201, [1000, 4099, 77, 1, 1024, 0])
    dev, sc, bm, dots = run_full_scan(fx, pl, wl)
    s = wl.signs()
    for t in range(wl.nq):
        n = int(wl.n_vis[t])
        if n == 0:
            assert np.isnan(sc[t]).all() and np.isnan(bm[t]).all()
            continue
        kc, ks = oracle.quantize(wl.keys(t), s)
        qc, qs = oracle.quantize(wl.q(0, [t])[0], s)
        I, A, D = oracle.score_rows(qc, qs, wl.w(0, [t])[0], kc, ks, want_dots=True)
        for j in range(32):
            for e in range(0, n, 97):
                _, exact, _ = oracle.head_dot(qc[j], qs[j], kc[e], ks[e])
                assert exact
        assert np.array_equal(dots[t, :, :n].astype(np.float64), D), f"query {t}: per-head dots differ"
        assert_scores_close(sc[t, :n], I, A, f"query {t}")
        assert np.isnan(sc[t, n:]).all(), "scores written past n"
        nb = (n + 7) // 8
        ref_bm = oracle.block_max(I, 8)
        Ab = block_A(A, n)
        assert np.all(np.abs(bm[t, :nb] - ref_bm) <= TOL * np.maximum(Ab, 1e-30))
        assert np.isnan(bm[t, nb:]).all(), "block maxima written past ceil(n/8)"
        # the block maxima are exactly the maxima of the GPU's own scores
        pad = np.full(nb * 8, -np.inf, np.float32)
        pad[:n] = sc[t, :n]
        assert np.array_equal(bm[t, :nb], pad.reshape(nb, 8).max(axis=1))


def make_rows(rng, nq, n, kind):
    if kind == "normal":
        return rng.standard_normal((nq, n)).astype(np.float32)
    if kind == "ties":
        return rng.integers(-3, 4, (nq, n)).astype(np.float32)
    if kind == "equal":
        return np.full((nq, n), 1.5, np.float32)
    if kind == "neginf":
        a = rng.standard_normal((nq, n)).astype(np.float32)
        a[rng.random((nq, n)) < 0.7] = -np.inf
        return a
    raise KeyError(kind)


@pytest.mark.parametrize("n,k,kind", [(1000, 512, "normal"), (70000, 512, "normal"), (5000, 2048, "ties"),
                                      (3000, 7, "ties"), (20000, 512, "equal"), (9000, 2048, "neginf"),
                                      (300, 512, "normal"), (1 << 20, 512, "normal"), (1, 1, "normal"),
                                      # block-size boundaries of the short-row kernel (256 / 512 / 1024
                                      # threads), and candidate lists beyond the smaller LDS list
                                      (4096, 512, "normal"), (4097, 512, "normal"), (8192, 2048, "normal"),
                                      (8193, 512, "ties"), (4096, 2048, "equal"), (4000, 512, "ties"),
                                      # long rows whose bound admits every value (k large for the row),
                                      # so the candidates exceed what the finishing block stages in LDS
                                      (20000, 2048, "normal"), (33000, 2048, "neginf"), (16385, 1, "ties"),
                                      # k above 64 per wavefront: the bound from the lanes' fourth-largest
                                      # values, candidates beyond the smaller list
                                      (16384, 2048, "normal"), (12000, 2048, "ties"), (16384, 1500, "neginf"),
                                      (16384, 1025, "equal")])
def test_topk_exact(fx, n, k, kind):
    rng = np.random.default_rng(n + k)
    nq = 3
    vals = make_rows(rng, nq, n, kind)
    nvalid = np.array([n, max(n // 2, 0), max(n - 1, 0)], dtype=np.int32)
    ws = fx.workspace(fx.IDX_OP_TOPK, nq, n, k)
    out = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    oval = torch.empty((nq, k), dtype=torch.float32, device="cuda")
    fx.idx_topk(torch.from_numpy(vals).cuda(), n, k, out, ws, n_valid=torch.from_numpy(nvalid).cuda(), out_val=oval)
    torch.cuda.synchronize()
    out, oval = out.cpu().numpy(), oval.cpu().numpy()
    for t in range(nq):
        ref = oracle.topk(vals[t, :nvalid[t]].astype(np.float64), k)
        cnt = int((ref >= 0).sum())
        ref_pos = np.sort(ref[:cnt])  # the library reports the selected set in ascending position order
        assert np.array_equal(out[t, :cnt], ref_pos), f"row {t}"
        assert (out[t, cnt:] == -1).all()
        assert np.array_equal(oval[t, :cnt], vals[t, ref_pos])
        assert np.all(np.isneginf(oval[t, cnt:]))


def adversarial_rows(rng, nq, n, kind, k):
    """rows aimed at the candidate bound and the list passes of the selection"""
    if kind == "posinf_few":  # fewer +inf than k: counted before the passes
        a = rng.standard_normal((nq, n)).astype(np.float32)
        a[:, rng.choice(n, size=min(n, max(1, k // 3)), replace=False)] = np.inf
        return a
    if kind == "posinf_many":  # more +inf than k: positions decide among them
        a = rng.standard_normal((nq, n)).astype(np.float32)
        a[:, rng.choice(n, size=min(n, 2 * k + 3), replace=False)] = np.inf
        return a
    if kind == "nan":
        a = rng.standard_normal((nq, n)).astype(np.float32)
        a[rng.random((nq, n)) < 0.2] = np.nan
        return a
    if kind == "signed_zeros":  # -0 and +0 tie; a few positives and negatives around them
        a = np.where(rng.random((nq, n)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        m = rng.random((nq, n))
        a[m < k / (4 * n)] = 1.0
        a[(m > 0.5) & (m < 0.6)] = -1.0
        return a
    if kind == "narrow":  # keys that differ only in the low mantissa bits
        return (np.float32(3.0) + rng.integers(0, 300, (nq, n)).astype(np.float32) * np.float32(2.0 ** -20))
    if kind == "sparse":  # mostly -inf: few eligible values, spread over the row
        a = np.full((nq, n), -np.inf, np.float32)
        idx = rng.choice(n, size=min(n, 3 * k), replace=False)
        a[:, idx] = rng.standard_normal(len(idx)).astype(np.float32)
        return a
    if kind == "one_hot":  # a single huge value among ties
        a = np.zeros((nq, n), np.float32)
        a[:, n // 3] = 1e30
        return a
    if kind == "ties_below_k":  # fewer than k values above a value most of the row ties at
        a = np.ones((nq, n), np.float32)
        a[:, rng.choice(n, size=min(n, k // 2), replace=False)] = 5.0
        return a
    if kind == "ties_above_k":  # more than k values above a value most of the row ties at
        a = np.ones((nq, n), np.float32)
        a[:, rng.choice(n, size=min(n, k + 100), replace=False)] = rng.uniform(2.0, 3.0, min(n, k + 100))
        return a
    if kind == "ties_stacked":  # three tied levels: the top one clustered at the row start, so that
        a = np.ones((nq, n), np.float32)  # some wavefronts bound below it and rounds of ties follow
        a[rng.random((nq, n)) < 0.37] = 2.0
        a[:, :min(n, 5000)] = 3.0
        return a
    raise KeyError(kind)


@pytest.mark.parametrize("kind", ["posinf_few", "posinf_many", "nan", "signed_zeros", "narrow", "sparse", "one_hot",
                                  "ties_below_k", "ties_above_k", "ties_stacked"])
@pytest.mark.parametrize("n,k", [(16384, 512), (5000, 1025), (3000, 1), (70000, 512), (200000, 2048), (40000, 64),
                                 (16384, 2048)])
def test_topk_adversarial(fx, n, k, kind):
    rng = np.random.default_rng(zlib.crc32(f"{n},{k},{kind}".encode()))
    nq = 2
    vals = adversarial_rows(rng, nq, n, kind, k)
    nvalid = np.array([n, max(1, n - 37)], dtype=np.int32)
    ws = fx.workspace(fx.IDX_OP_TOPK, nq, n, k)
    out = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    oval = torch.empty((nq, k), dtype=torch.float32, device="cuda")
    for _ in range(2):  # the second call reuses the workspace as the first left it
        fx.idx_topk(torch.from_numpy(vals).cuda(), n, k, out, ws, n_valid=torch.from_numpy(nvalid).cuda(),
                    out_val=oval)
        torch.cuda.synchronize()
        o, ov = out.cpu().numpy(), oval.cpu().numpy()
        for t in range(nq):
            ref = oracle.topk(vals[t, :nvalid[t]].astype(np.float64), k)
            cnt = int((ref >= 0).sum())
            ref_pos = np.sort(ref[:cnt])
            assert np.array_equal(o[t, :cnt], ref_pos), f"row {t}"
            assert (o[t, cnt:] == -1).all()
            assert np.array_equal(ov[t, :cnt], vals[t, ref_pos])  # -0 == +0
            assert np.all(np.isneginf(ov[t, cnt:]))


@pytest.mark.parametrize("n,k", [(4096, 512), (8000, 512), (16384, 512)])
def test_topk_many_rows(fx, n, k):
    # many rows per launch (the prefill shape), each with its own valid length
    rng = np.random.default_rng(n * 7 + k)
    nq = 777
    vals = rng.standard_normal((nq, n)).astype(np.float32)
    nvalid = rng.integers(0, n + 1, nq).astype(np.int32)
    nvalid[:3] = [n, 0, k - 1]
    ws = fx.workspace(fx.IDX_OP_TOPK, nq, n, k)
    out = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    fx.idx_topk(torch.from_numpy(vals).cuda(), n, k, out, ws, n_valid=torch.from_numpy(nvalid).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for t in range(nq):
        ref = oracle.topk(vals[t, :nvalid[t]].astype(np.float64), k)
        cnt = int((ref >= 0).sum())
        assert np.array_equal(out[t, :cnt], np.sort(ref[:cnt])), f"row {t}"
        assert (out[t, cnt:] == -1).all(), f"row {t}"


@pytest.mark.parametrize("n,kind", [(16384 * 8, "equal"), (16385 * 8, "equal"), (1 << 20, "equal"),
                                    (1 << 20, "few_distinct"), (1 << 20, "ties_below_k"), (100003, "ties_above_k")])
def test_build_pool_ties(fx, n, kind):
    """pools over rows of tied block maxima (a zero query gives all-equal rows): equal to the
    oracle's full sort with ties to the lower block id, on both selection paths"""
    rng = np.random.default_rng(n + len(kind))
    nq = 3
    nb = (n + 7) // 8
    if kind == "equal":
        bm = np.zeros((nq, nb), np.float32)
    elif kind == "few_distinct":
        bm = rng.integers(0, 97, (nq, nb)).astype(np.float32)
    elif kind == "ties_below_k":
        bm = np.ones((nq, nb), np.float32)
        for t in range(nq):
            bm[t, rng.choice(nb, size=1000, replace=False)] = 4.0
    else:
        bm = np.ones((nq, nb), np.float32)
        for t in range(nq):
            bm[t, rng.choice(nb, size=3000, replace=False)] = rng.uniform(2, 3, 3000)
    nv = np.array([n, n - 5, (n * 3) // 4], np.int32)
    ws = fx.workspace(fx.IDX_OP_BUILD_POOL, nq, n, 2048)
    pb = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    pc = torch.empty(nq, dtype=torch.int32, device="cuda")
    fx.idx_build_pool(torch.from_numpy(bm).cuda(), torch.from_numpy(nv).cuda(), n, pb, pc, ws)
    torch.cuda.synchronize()
    pb, pc = pb.cpu().numpy(), pc.cpu().numpy()
    for t in range(nq):
        nbt = (int(nv[t]) + 7) // 8
        ref = oracle.pool(bm[t, :nbt].astype(np.float64), int(nv[t]), 8, 2048)
        assert pc[t] == len(ref), (t, pc[t], len(ref))
        assert np.array_equal(pb[t, :len(ref)], ref), t
        assert (pb[t, len(ref):] == -1).all()


@pytest.mark.parametrize("n", [1, 8, 9, 16383, 16384, 16385, 16392, 100003, 1 << 20])
def test_build_pool_exact(fx, n):
    rng = np.random.default_rng(n)
    nq = 2
    nb = (n + 7) // 8
    bm = rng.standard_normal((nq, nb)).astype(np.float32)
    bm[1] = np.round(bm[1])  # ties
    nv = np.array([n, n], np.int32)
    ws = fx.workspace(fx.IDX_OP_BUILD_POOL, nq, n, 2048)
    pb = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    pc = torch.empty(nq, dtype=torch.int32, device="cuda")
    bm_d, nv_d = torch.from_numpy(bm).cuda(), torch.from_numpy(nv).cuda()
    fx.idx_build_pool(bm_d, nv_d, n, pb, pc, ws)
    torch.cuda.synchronize()
    pb2 = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    fx.idx_build_pool(bm_d, nv_d, n, pb2, pc, ws)  # reuse without clearing
    torch.cuda.synchronize()
    assert torch.equal(pb, pb2)
    pb, pc = pb.cpu().numpy(), pc.cpu().numpy()
    for t in range(nq):
        ref = oracle.pool(bm[t].astype(np.float64), n, 8, 2048)
        assert pc[t] == len(ref)
        assert np.array_equal(pb[t, :len(ref)], ref)
        assert (pb[t, len(ref):] == -1).all()


@pytest.mark.parametrize("n,k", [(1, 512), (9, 512), (4096 * 8, 512), (4097 * 8 + 3, 512), (131072 * 8 + 5, 512),
                                 (300001, 2048), (1 << 20, 7)])
def test_top_blocks_exact(fx, n, k):
    """idx_top_blocks: the k largest raw block maxima (ties to the lower block id, no pin),
    ascending ids and counts, against the oracle's full-sort top-k over the block maxima."""
    rng = np.random.default_rng(n + k)
    nq = 3
    nb = (n + 7) // 8
    bm = rng.standard_normal((nq, nb)).astype(np.float32)
    bm[1] = np.round(bm[1])  # ties
    bm[2, ::3] = -np.inf  # blocks that can never be selected
    nv = np.array([n, n, n], np.int32)
    ws = fx.workspace(fx.IDX_OP_BUILD_POOL, nq, n, k)
    out = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
    fx.idx_top_blocks(torch.from_numpy(bm).cuda(), torch.from_numpy(nv).cuda(), n, k, out, cnt, ws)
    torch.cuda.synchronize()
    out, cnt = out.cpu().numpy(), cnt.cpu().numpy()
    for t in range(nq):
        ref = oracle.topk(bm[t].astype(np.float64), k)
        ref = np.sort(ref[ref >= 0])
        assert cnt[t] == len(ref), (t, cnt[t], len(ref))
        assert np.array_equal(out[t, :len(ref)], ref), t
        assert (out[t, len(ref):] == -1).all()


def test_gather_matches_full_scan(fx, pl):
    wl = synth.decode_workload("g", 202, [30000, 3001])
    dev, sc, bm, _ = run_full_scan(fx, pl, wl, want_dots=False)
    plan = pl.DecodePlan(dev)
    plan.q_codes[0], plan.q_scales[0] = fx.idx_quantize_q(dev.q[0], dev.signs)
    plan.block_max.copy_(torch.from_numpy(bm))
    plan.build_pool()
    plan.pool_select(0)
    torch.cuda.synchronize()
    pbk = plan.pool_blocks.cpu().numpy()
    pcn = plan.pool_count.cpu().numpy()
    ps = plan.pool_scores[0].cpu().numpy()
    for t in range(wl.nq):
        n = int(wl.n_vis[t])
        for i in range(plan.max_blocks):
            for r in range(8):
                slot = 8 * i + r
                if i < pcn[t] and 8 * pbk[t, i] + r < n:
                    assert ps[t, slot] == sc[t, 8 * pbk[t, i] + r]  # bit-identical arithmetic
                else:
                    assert np.isneginf(ps[t, slot])


@pytest.mark.parametrize("nq,max_blocks,stride", [(512, 1024, 1030), (256, 2100, 2100)])
def test_gather_long_form_lists(fx, nq, max_blocks, stride):
    """Launches of at least 2^22 slots (the prefill shape): one key cache shared by every query,
    ragged lengths, unsorted block lists with duplicates, negative ids, ids past the range, counts
    of zero, past max_blocks and negative. Every slot must equal the full scan's score of its
    position bit for bit, or be -inf."""
    n_keys = 20000
    rng = np.random.default_rng(nq + max_blocks)
    s = synth.signs(41)
    keys = synth.normal_bf16(41, 3, 0, 0, n_keys * 128).reshape(n_keys, 128)
    kc, ks = fx.idx_quantize_q(to_dev_bf16(keys), torch.from_numpy(s).cuda())
    q = synth.normal_bf16(41, 2, 0, 0, nq * 32 * 128).reshape(nq, 32, 128)
    qc, qs = fx.idx_quantize_q(to_dev_bf16(q), torch.from_numpy(s).cuda())
    w = torch.from_numpy(synth.normal_f32(41, 4, 0, 0, nq * 32, 32 ** -0.5).reshape(nq, 32)).cuda()
    n_vis = rng.integers(12000, n_keys + 1, nq).astype(np.int32)
    n_vis[:3] = [0, 1, n_keys]
    base = torch.zeros(nq, dtype=torch.int64, device="cuda")
    nv = torch.from_numpy(n_vis).cuda()
    scores = torch.full((nq, n_keys), float("nan"), device="cuda")
    fx.idx_score_full(kc, ks, base, nv, qc, qs, w, n_keys, scores=scores)
    nb_max = (n_keys + 7) // 8
    blocks = rng.integers(-3, nb_max + 5, (nq, stride)).astype(np.int32)
    blocks[1::3, :max_blocks // 2] = np.sort(rng.choice(nb_max, (len(blocks[1::3]), max_blocks // 2)), axis=1)
    counts = rng.integers(0, max_blocks + 1, nq).astype(np.int32)
    counts[3:9] = [0, max_blocks, max_blocks + 50, -4, 1, max_blocks - 1]
    out = torch.full((nq, 8 * max_blocks + 16), float("nan"), device="cuda")
    fx.idx_score_pool_gather(kc, ks, base, nv, torch.from_numpy(blocks).cuda(), torch.from_numpy(counts).cuda(),
                             max_blocks, qc, qs, w, out)
    torch.cuda.synchronize()
    sc, got = scores.cpu().numpy(), out.cpu().numpy()
    assert np.isnan(got[:, 8 * max_blocks:]).all()  # nothing written past the slots
    got = got[:, :8 * max_blocks]
    cnt = np.clip(counts, 0, max_blocks)
    b = blocks[:, :max_blocks].astype(np.int64)
    pos = (8 * b[:, :, None] + np.arange(8)).reshape(nq, -1)
    ent = np.repeat(np.arange(max_blocks), 8)[None, :]
    valid = (ent < cnt[:, None]) & (np.repeat(b, 8, axis=1) >= 0) & (pos < n_vis[:, None])
    want = np.where(valid, sc[np.arange(nq)[:, None], np.where(valid, pos, 0)], -np.inf)
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_recorded_decode_step_equals_run(fx, pl):
    """DecodePlan.compiled(): the recorded step, replayed twice, leaves every output equal to run()'s"""
    wl = synth.decode_workload("rec", 77, [30000, 3001, 100000], layers=2)
    dev = pl.DeviceWorkload.from_workload(wl)
    a = pl.DecodePlan(dev)
    a.run()
    b = pl.DecodePlan(dev)
    rep = b.compiled()
    rep()
    rep()
    torch.cuda.synchronize()
    assert torch.equal(a.pool_blocks, b.pool_blocks) and torch.equal(a.pool_count, b.pool_count)
    for layer in range(a.layers + 1):
        assert torch.equal(a.topk[layer], b.topk[layer])
        assert torch.equal(a.topk_val[layer], b.topk_val[layer])


def check_decode(fx, pl, wl, k=512):
    dev = pl.DeviceWorkload.from_workload(wl)
    out = pl.decode_step(dev, k=k)
    torch.cuda.synchronize()
    s = wl.signs()
    top = out["topk"].cpu().numpy()
    pbk, pcn = out["pool_blocks"].cpu().numpy(), out["pool_count"].cpu().numpy()
    rtop = [r.cpu().numpy() for r in out["reindex_topk"]]
    for t in range(wl.nq):
        n = int(wl.n_vis[t])
        kc, ks = oracle.quantize(wl.keys(t), s)
        qc, qs = oracle.quantize(wl.q(0, [t])[0], s)
        I, A = oracle.score_rows(qc, qs, wl.w(0, [t])[0], kc, ks)
        assert_topk_set(top[t], I, A, k, f"full top-k q{t}")
        bm = oracle.block_max(I, 8)
        gpool = pbk[t, :pcn[t]]
        assert_pool_set(gpool, bm, block_A(A, n), n, 2048, f"pool q{t}")
        pos = set()
        for b in gpool:
            pos.update(range(8 * b, min(8 * b + 8, n)))
        assert set(int(x) for x in top[t] if x >= 0) <= pos, "Full top-k must lie in the pool"
        for li in range(wl.layers):
            qc2, qs2 = oracle.quantize(wl.q(li + 1, [t])[0], s)
            I2, A2 = oracle.score_rows(qc2, qs2, wl.w(li + 1, [t])[0], kc, ks)
            # Reindex in the GPU's own pool (mask form); the pool itself is checked above
            masked = np.full(n, -np.inf)
            idx = np.array(sorted(pos), dtype=np.int64)
            masked[idx] = I2[idx]
            assert_topk_set(rtop[li][t], masked, A2, k, f"reindex layer {li + 1} q{t}")
            assert set(int(x) for x in rtop[li][t] if x >= 0) <= pos


def test_decode_32k_full_size(fx, pl):
    check_decode(fx, pl, synth.config("decode_32k"))


def test_decode_ragged_batch(fx, pl):
    check_decode(fx, pl, synth.decode_workload("r", 203, [20001, 5000, 700, 16384, 16385, 9], layers=2))


def test_decode_ragged_batch_long_pool(fx, pl):
    # rows past 16384 blocks send the whole batch's pool through the long-row selection (bound,
    # collect, finish), short and empty rows included
    check_decode(fx, pl, synth.decode_workload("rl", 207, [300000, 9, 0, 140000, 131073, 1000], layers=1))


@pytest.mark.parametrize("n_keys,nq", [(6000, 48), (4100, 8), (700, 64), (300, 20)])
def test_prefill_parity(fx, pl, n_keys, nq):
    # chunked prefill end to end; the small caches leave queries with fewer than 512 blocks (every
    # block kept) and, at 300 keys, fewer than 512 visible keys (all of them selected, then -1)
    wl = synth.prefill_workload("pf", 204 + n_keys, n_keys, nq)
    dev = pl.DeviceWorkload.from_workload(wl, group=nq)
    plan = pl.PrefillPlan(dev).run()
    torch.cuda.synchronize()
    top = plan.topk.cpu().numpy()
    s = wl.signs()
    kc, ks = oracle.quantize(wl.keys(0), s)
    for t in list(range(0, wl.nq, 5)) + [wl.nq - 1]:
        n = int(wl.n_vis[t])
        qc, qs = oracle.quantize(wl.q(0, [t])[0], s)
        I, A = oracle.score_rows(qc, qs, wl.w(0, [t])[0], kc[:n], ks[:n])
        assert_topk_set(top[t], I, A, 512, f"prefill q{t}")


@pytest.mark.parametrize("nblocks,k", [(300, 512), (2048, 512), (4096, 2048), (2048, 100)])
def test_topk_with_block_map(fx, nblocks, k):
    # slot s stands for position 8 * map[s // 8] + s % 8; ties break on the mapped position
    rng = np.random.default_rng(nblocks + k)
    nq = 2
    slots = nblocks * 8
    vals = rng.integers(-5, 6, (nq, slots)).astype(np.float32)
    vals[:, rng.random(slots) < 0.1] = -np.inf
    maps = np.stack([rng.permutation(50000)[:nblocks] for _ in range(nq)]).astype(np.int32)
    ws = fx.workspace(fx.IDX_OP_TOPK, nq, slots, k)
    out = torch.empty((nq, k), dtype=torch.int32, device="cuda")
    fx.idx_topk(torch.from_numpy(vals).cuda(), slots, k, out, ws, blocks=torch.from_numpy(maps).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for t in range(nq):
        pos = (8 * maps[t][:, None] + np.arange(8)[None, :]).reshape(-1)
        full = np.full(int(pos.max()) + 1, -np.inf)
        full[pos] = vals[t]
        ref = oracle.topk(full, k)
        cnt = int((ref >= 0).sum())
        assert sorted(out[t, :cnt].tolist()) == sorted(ref[:cnt].tolist()), f"row {t}"
        assert (out[t, cnt:] == -1).all()


@pytest.mark.parametrize("outputs", ["both", "block_max", "scores"])
@pytest.mark.parametrize("n_keys,nqs,group", [(6000, 48, 48), (3000, 37, 37), (20000, 70, 35), (9000, 16, 16),
                                              # groups that leave query slots of the last block of a group empty
                                              (7000, 30, 6), (5000, 10, 5), (3000, 9, 3), (12000, 36, 6)])
def test_multi_query_scan_matches_single_query(fx, pl, n_keys, nqs, group, outputs):
    # the many-query scan (group > 1) must reproduce the per-query scan bit for bit when scores
    # are written, and its block maxima alone within the scores' tolerance (another fp32 order of
    # the same exact head terms), for each combination of requested outputs (untouched entries stay
    # NaN on both sides)
    wl = synth.prefill_workload("mq", 205 + nqs, n_keys, nqs)
    dev = pl.DeviceWorkload.from_workload(wl, group=group)
    if group < nqs:  # several groups over the same keys, each with its own causal bounds
        dev.n_vis = torch.cat([dev.n_vis[:group] - 1000 * i for i in range(nqs // group)])
    qc, qs = fx.idx_quantize_q(dev.q[0], dev.signs)
    nb = (dev.max_n + 7) // 8
    want_sc = outputs in ("both", "scores")
    want_bm = outputs in ("both", "block_max")
    outs = []
    for g in (1, group):
        sc = torch.full((wl.nq, dev.max_n), float("nan"), device="cuda")
        bm = torch.full((wl.nq, nb), float("nan"), device="cuda")
        fx.idx_score_full(dev.k_codes, dev.k_scales, dev.k_base, dev.n_vis, qc, qs, dev.w[0], dev.max_n, group=g,
                          scores=sc if (g == 1 or want_sc) else None, block_max=bm if (g == 1 or want_bm) else None)
        outs.append((sc, bm))
    torch.cuda.synchronize()
    if want_sc:
        assert torch.equal(torch.nan_to_num(outs[0][0], nan=7.0), torch.nan_to_num(outs[1][0], nan=7.0))
    if want_bm and want_sc:
        assert torch.equal(torch.nan_to_num(outs[0][1], nan=7.0), torch.nan_to_num(outs[1][1], nan=7.0))
    elif want_bm:
        # single-query block maxima bound the many-query ones within 1e-5 of A: A >= |I| for every
        # score (A sums |w_j| ReLU(d_j)), so compare against the single query's amplitude bound
        # taken from the oracle on each block's winning key
        a, b = outs[0][1].cpu().numpy(), outs[1][1].cpu().numpy()
        assert np.array_equal(np.isnan(a), np.isnan(b))
        assert np.array_equal(np.isneginf(a), np.isneginf(b))
        fin = np.isfinite(a)
        s_np = wl.signs()
        kc, ks = oracle.quantize(wl.keys(0), s_np)
        for t in range(wl.nq):
            nbt = int(fin[t].sum())
            if nbt == 0:
                continue
            n = int(dev.n_vis[t])
            qcn, qsn = oracle.quantize(wl.q(0, [t])[0], s_np)
            I, A = oracle.score_rows(qcn, qsn, wl.w(0, [t])[0], kc[:n], ks[:n])
            pad = np.full((nbt * 8 - n), -np.inf)
            Ib = np.concatenate([I, pad]).reshape(nbt, 8)
            Ab = np.concatenate([A, np.zeros(nbt * 8 - n)]).reshape(nbt, 8)
            tol = 1e-5 * Ab.max(axis=1)
            assert np.all(np.abs(b[t, :nbt] - Ib.max(axis=1)) <= tol), t
            assert np.all(np.abs(a[t, :nbt] - Ib.max(axis=1)) <= tol), t
    # nothing beyond a query's visible blocks is written
    nvis = dev.n_vis.cpu().numpy()
    for t in range(wl.nq):
        nbt = (int(nvis[t]) + 7) // 8
        if want_bm:
            assert torch.isnan(outs[1][1][t, nbt:]).all(), f"block max written past query {t}"
        if want_sc:
            assert torch.isnan(outs[1][0][t, int(nvis[t]):]).all(), f"score written past query {t}"
