"""Helpers shared by the GPU parity tests: oracle references and set comparisons with the
boundary tolerance. Imported by tests only."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

TOL = 1e-5  # relative tolerance on scores, against A = sum_j |w_j| ReLU(d_j)


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def oracle_keys(wl, b, s):
    kc, ks = oracle.quantize(wl.keys(b), s)
    return kc, ks


def assert_scores_close(got, ref, A, what=""):
    got = np.asarray(got, dtype=np.float64)
    bad = np.abs(got - ref) > TOL * np.maximum(A, 1e-30)
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} scores out of tolerance, first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} A {A[i]!r}")


def assert_topk_set(got_idx, I_ref, A_ref, k, what=""):
    """GPU top-k index set equals the oracle's, except entries within tolerance of the k-th score."""
    got = [int(x) for x in got_idx if x >= 0]
    eligible = np.isfinite(I_ref)
    n_el = int(eligible.sum())
    assert len(got) == min(k, n_el), f"{what}: selected {len(got)} of expected {min(k, n_el)}"
    assert len(set(got)) == len(got), f"{what}: duplicate indices"
    ref = oracle.topk(I_ref, k)
    ref = [int(x) for x in ref if x >= 0]
    if n_el <= k:
        assert set(got) == set(ref), f"{what}: short row must select every eligible entry"
        return
    b = I_ref[ref[-1]]
    for s in set(got) ^ set(ref):
        excuse = TOL * max(abs(b), A_ref[s])
        assert abs(I_ref[s] - b) <= excuse, f"{what}: index {s} score {I_ref[s]!r} vs boundary {b!r}"


def assert_pool_set(got_blocks, bm_ref, A_block, n, keep=2048, what=""):
    """pool block set equals the oracle's up to blocks within tolerance of the keep-th block value."""
    got = sorted(int(x) for x in got_blocks if x >= 0)
    ref = oracle.pool(bm_ref, n, 8, keep).tolist()
    assert len(got) == len(ref), f"{what}: pool size {len(got)} vs {len(ref)}"
    assert got == sorted(got), f"{what}: pool not ascending"
    if set(got) == set(ref):
        return
    nb = (n + 7) // 8
    last = (n - 1) // 8
    vals = np.where(np.arange(nb) == last, np.inf, bm_ref)
    order = sorted(range(nb), key=lambda b: (-vals[b], b))
    bnd = vals[order[keep - 1]]
    for b in set(got) ^ set(ref):
        assert abs(vals[b] - bnd) <= TOL * max(abs(bnd), A_block[b]), f"{what}: block {b} {vals[b]!r} vs {bnd!r}"


def block_A(A, n):
    nb = (n + 7) // 8
    pad = np.zeros(nb * 8)
    pad[:n] = A
    return pad.reshape(nb, 8).max(axis=1)
