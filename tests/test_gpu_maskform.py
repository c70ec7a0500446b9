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


def check_mask_equals_gather(pl, wl):
    dev = pl.DeviceWorkload.from_workload(wl)
    gather = pl.DecodePlan(dev).run()
    mask = pl.MaskFormPlan(dev).run()
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


def test_mask_form_equals_gather_form_ragged(fx, pl):
    check_mask_equals_gather(pl, synth.decode_workload("mf", 211, [20001, 5000, 700, 16384, 16385, 9, 40000],
                                                       layers=3))


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
