"""The pool's training form on the GPU: the mask step bit-exact against the oracle's, and the
mask-form decode step (every layer scores every visible position, the pool masks the rest)
against the gather form, which the decode parity tests pin to the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

NEG = np.float32(-np.inf)


@pytest.fixture(scope="module")
def fx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_fp4_lightning_amd

    return top_fp4_lightning_amd


@pytest.fixture(scope="module")
def pl(fx):
    from top_fp4_lightning_amd import pipeline

    return pipeline


def mask_case(seed, n_vis, max_n, group, stride_pad=3, pool_stride=2048):
    """Rows of seeded fp32 values, one pool per `group` rows: sorted or shuffled block ids with
    duplicates, ids past the row and negative ids, and counts that clamp."""
    rng = np.random.default_rng(seed)
    nq = len(n_vis)
    rows = rng.standard_normal((nq, max_n + stride_pad)).astype(np.float32)
    npool = nq // group
    pools = np.full((npool, pool_stride), -1, dtype=np.int32)
    counts = np.zeros(npool, dtype=np.int32)
    for p in range(npool):
        nb = (max(int(n_vis[p * group: (p + 1) * group].max()), 1) + 7) // 8
        c = int(rng.integers(0, pool_stride + 1))
        ids = rng.integers(-3, nb + 5, size=c).astype(np.int32)
        if p % 2 == 0:
            ids.sort()
        pools[p, :c] = ids
        counts[p] = c if p % 3 else c + 7  # counts past pool_stride clamp to it
    return rows, pools, counts


@pytest.mark.parametrize("n_vis,max_n,group", [
    ([1000, 0, 8, 9, 16384, 16385, 40000, 50000], 50000, 1),
    ([70000, 69999, 65536, 1], 70000, 2),
    ([5, 300000, 12, 8], 300000, 4),
    ([33, 100], 90, 1),  # n_vis above max_n clamps to it
])
def test_mask_pool_bit_exact(fx, n_vis, max_n, group):
    rows, pools, counts = mask_case(len(n_vis) * 7 + group, np.array(n_vis), max_n, group)
    d = torch.from_numpy(rows).cuda()
    before = d.clone()
    nv = torch.tensor(n_vis, dtype=torch.int32, device="cuda")
    fx.idx_mask_pool(d[:, :], nv, max_n, torch.from_numpy(pools).cuda(), torch.from_numpy(counts).cuda(),
                     group=group)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    for t, n in enumerate(n_vis):
        n = min(n, max_n)
        p = t // group
        c = min(int(counts[p]), pools.shape[1])
        want = oracle.mask_pool(rows[t, :n].astype(np.float64), pools[p, :c]).astype(np.float32)
        assert np.array_equal(got[t, :n].view(np.uint32), want.view(np.uint32)), f"row {t} n={n}"
        assert np.array_equal(got[t, n:], before[t, n:].cpu().numpy()), f"row {t}: past n_vis must not change"


def topk_pool_case(seed, n_vis, max_n, group, max_blocks, pool_stride, ties):
    """Seeded rows (optionally few distinct values with -0 among them, so that ties decide) and one
    pool per `group` rows: distinct block ids, some outside the row, ascending in even pools and
    shuffled in odd ones, counts that run into the -1 padding or past max_blocks."""
    rng = np.random.default_rng(seed)
    nq = len(n_vis)
    rows = rng.standard_normal((nq, max_n + 3)).astype(np.float32)
    if ties:
        rows = (np.round(rows * 2) / 2).astype(np.float32)
    npool = nq // group
    pools = np.full((npool, pool_stride), -1, dtype=np.int32)
    counts = np.zeros(npool, dtype=np.int32)
    for p in range(npool):
        nb = (max(int(max(n_vis[p * group: (p + 1) * group])), 1) + 7) // 8
        span = np.arange(-3, nb + 5, dtype=np.int32)
        c = int(rng.integers(0, min(pool_stride, len(span)) + 1))
        ids = rng.choice(span, size=c, replace=False).astype(np.int32)
        if p % 2 == 0:
            ids.sort()
        pools[p, :c] = ids
        counts[p] = c + (7 if p % 3 == 0 else 0)
    return rows, pools, counts


@pytest.mark.parametrize("n_vis,max_n,group,max_blocks,k,ties", [
    ([1000, 0, 8, 9, 16384, 16385, 40000, 50000], 50000, 1, 2048, 512, False),
    ([70000, 69999, 65536, 1], 70000, 2, 2048, 512, True),
    ([5, 300000, 12, 8], 300000, 4, 2048, 512, False),
    ([3000, 2001, 777, 64], 3000, 1, 100, 300, True),  # narrow pool, counts past max_blocks clamp
    ([20000, 19999], 20000, 1, 2048, 2048, False),  # k = 2048: more than half of a full pool
    ([33, 100], 90, 2, 16, 7, False),  # n_vis above max_n clamps to it
])
def test_topk_pool_against_oracle(fx, n_vis, max_n, group, max_blocks, k, ties):
    """idx_topk_pool is the oracle's mask-then-top-k: same positions (ascending for ascending
    pools), the scores at them, -1 / -inf after them."""
    rows, pools, counts = topk_pool_case(len(n_vis) * 11 + group + k, n_vis, max_n, group, max_blocks,
                                         max(max_blocks, 64), ties)
    nq = len(n_vis)
    d = torch.from_numpy(rows).cuda()
    nv = torch.tensor(n_vis, dtype=torch.int32, device="cuda")
    out = torch.full((nq, k + 5), 77, dtype=torch.int32, device="cuda")
    val = torch.full((nq, k + 5), 77.0, dtype=torch.float32, device="cuda")
    fx.idx_topk_pool(d, nv, max_n, torch.from_numpy(pools).cuda(), torch.from_numpy(counts).cuda(), max_blocks, k,
                     out, out_val=val, group=group)
    torch.cuda.synchronize()
    got, gv = out.cpu().numpy(), val.cpu().numpy()
    assert (got[:, k:] == 77).all() and (gv[:, k:] == 77.0).all(), "wrote past k"
    for t, n in enumerate(n_vis):
        n = min(n, max_n)
        p = t // group
        ids = pools[p, :min(int(counts[p]), max_blocks)]
        ref = oracle.reindex_mask(rows[t, :n].astype(np.float64), ids, 8, k)
        want = [int(x) for x in ref if x >= 0]
        sel = [int(x) for x in got[t, :k] if x >= 0]
        what = f"row {t} n={n} pool {p} ({len(ids)} ids)"
        assert len(sel) == len(want), what
        assert (got[t, len(sel):k] == -1).all() and np.isneginf(gv[t, len(sel):k]).all(), what
        if p % 2 == 0:
            assert sel == sorted(want), what
        else:
            assert sorted(sel) == sorted(want), what
        v = rows[t, sel] + np.float32(0.0)  # a selected -0 is reported as +0
        assert np.array_equal(gv[t, :len(sel)].view(np.uint32), v.view(np.uint32)), what


def test_topk_pool_equals_mask_then_topk(fx):
    """The fused call and the literal form (in-place mask, then a top-k over whole rows, the long-row
    path) give the same bits, on rows longer than one selection block."""
    n_vis = [200000, 131073, 16385, 90000]
    max_n = 200000
    rows, pools, counts = topk_pool_case(5, n_vis, max_n, 2, 2048, 2048, False)
    pools = np.sort(np.where(pools < 0, np.iinfo(np.int32).max, pools), axis=1)  # ascending, padding last
    pools[pools == np.iinfo(np.int32).max] = -1
    d = torch.from_numpy(rows).cuda()
    nv = torch.tensor(n_vis, dtype=torch.int32, device="cuda")
    pb, pc = torch.from_numpy(pools).cuda(), torch.from_numpy(counts).cuda()
    o1 = torch.empty(4, 512, dtype=torch.int32, device="cuda")
    v1 = torch.empty(4, 512, dtype=torch.float32, device="cuda")
    fx.idx_topk_pool(d, nv, max_n, pb, pc, 2048, 512, o1, out_val=v1, group=2)
    fx.idx_mask_pool(d, nv, max_n, pb, pc, group=2)
    o2 = torch.empty_like(o1)
    v2 = torch.empty_like(v1)
    ws = fx.workspace(fx.IDX_OP_TOPK, 4, max_n, 512)
    fx.idx_topk(d, max_n, 512, o2, ws, n_valid=nv, out_val=v2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(v1.view(torch.int32), v2.view(torch.int32))


def check_mask_equals_gather(pl, wl, write_mask=False):
    dev = pl.DeviceWorkload.from_workload(wl)
    gather = pl.DecodePlan(dev).run()
    mask = pl.MaskFormPlan(dev, write_mask=write_mask).run()
    torch.cuda.synchronize()
    assert torch.equal(mask.pool_count, gather.pool_count)
    for t in range(dev.nq):
        c = int(gather.pool_count[t])
        assert torch.equal(mask.pool_blocks[t, :c], gather.pool_blocks[t, :c]), f"pool q{t}"
    for layer in range(mask.L):
        mi, mv = mask.layer_topk(layer)
        assert torch.equal(mi, gather.topk[layer]), f"layer {layer} top-k indices"
        sel = mi >= 0
        assert torch.equal(mv[sel], gather.topk_val[layer][sel]), f"layer {layer} top-k values"


@pytest.mark.parametrize("write_mask", [False, True])
def test_mask_form_equals_gather_form_ragged(fx, pl, write_mask):
    check_mask_equals_gather(pl, synth.decode_workload("mf", 211, [20001, 5000, 700, 16384, 16385, 9, 40000],
                                                       layers=3), write_mask)


def test_mask_form_equals_gather_form_spec_decode(fx, pl):
    check_mask_equals_gather(pl, synth.spec_decode_workload("mfs", 212, [30000, 17000], positions=3, layers=2))


def test_mask_form_against_oracle(fx, pl):
    """Directly against the oracle's training form: full scores of each layer, its pool, the mask
    and the top-512, on a workload whose rows span several pool chunks."""
    from parity import assert_topk_set

    wl = synth.decode_workload("mfo", 213, [24001, 3000], layers=2)
    dev = pl.DeviceWorkload.from_workload(wl)
    plan = pl.MaskFormPlan(dev).run()
    torch.cuda.synchronize()
    s = wl.signs()
    for t in range(wl.nq):
        n = int(wl.n_vis[t])
        kc, ks = oracle.quantize(wl.keys(t), s)
        pb = plan.pool_blocks[t, :int(plan.pool_count[t])].cpu().numpy()
        for layer in range(plan.L):
            qc, qs = oracle.quantize(wl.q(layer, [t])[0], s)
            I, A = oracle.score_rows(qc, qs, wl.w(layer, [t])[0], kc, ks)
            idx, _ = plan.layer_topk(layer)
            assert_topk_set(idx[t].cpu().numpy(), oracle.mask_pool(I, pb), A, 512, f"layer {layer} q{t}")
