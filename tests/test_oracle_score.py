"""Pins for the oracle's per-head dot, score and MAC accounting (CPU only)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def e2m1_mags():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        return [Fraction(v) for v in [l for l in f if l.strip() and not l.startswith("#")][0].split()]


def dequant_exact(codes, scales):
    """exact rational values of one quantised 128-row, from the pages' value list."""
    mags = e2m1_mags()
    out = []
    for i in range(128):
        c = (int(codes[i // 2]) >> (4 * (i & 1))) & 15
        v = mags[c & 7] * (-1 if c & 8 else 1)
        out.append(v * Fraction(2) ** (int(scales[i // 32]) - 127))
    return out


def random_codes(rng, n):
    return rng.integers(0, 256, (n, 64), dtype=np.uint8)


@pytest.mark.parametrize("spread", [0, 3, 9, 30])
def test_head_dot_equals_exact_dequantised_dot(spread):
    rng = np.random.default_rng(100 + spread)
    for _ in range(200):
        qc, kc = random_codes(rng, 1)[0], random_codes(rng, 1)[0]
        qs = (127 + rng.integers(-spread // 2 - 1, spread // 2 + 1, 4)).astype(np.uint8)
        ks = (127 + rng.integers(-spread // 2 - 1, spread // 2 + 1, 4)).astype(np.uint8)
        d, exact, sp = oracle.head_dot(qc, qs, kc, ks)
        ref = sum(a * b for a, b in zip(dequant_exact(qc, qs), dequant_exact(kc, ks)))
        assert d == float(ref)
        rep = float(np.float32(float(ref))) == ref
        assert exact == rep


def test_head_dot_exact_on_workload_data():
    # the synthetic recipe keeps every per-head dot exactly representable in fp32 with a small
    # scale-exponent spread, which is the precondition for bit-exact MFMA results
    w = synth.decode_workload("t", 21, [600])
    s = w.signs()
    qc, qs = oracle.quantize(w.q(0, [0])[0], s)
    kc, ks = oracle.quantize(w.keys(0), s)
    worst = 0
    for j in range(32):
        for e in range(0, 600, 7):
            d, exact, sp = oracle.head_dot(qc[j], qs[j], kc[e], ks[e])
            assert exact
            worst = max(worst, sp)
    assert worst <= 9


def test_score_definition_bruteforce():
    w = synth.decode_workload("t", 22, [40])
    s = w.signs()
    qc, qs = oracle.quantize(w.q(0, [0])[0], s)
    kc, ks = oracle.quantize(w.keys(0), s)
    wt = w.w(0, [0])[0]
    I, A, dots = oracle.score_rows(qc, qs, wt, kc, ks, want_dots=True)
    for e in range(40):
        kv = dequant_exact(kc[e], ks[e])
        tot, tota = Fraction(0), Fraction(0)
        for j in range(32):
            d = sum(a * b for a, b in zip(dequant_exact(qc[j], qs[j]), kv))
            assert dots[j, e] == float(d)
            r = max(d, Fraction(0))
            tot += Fraction(float(wt[j])) * r
            tota += abs(Fraction(float(wt[j]))) * r
        assert abs(I[e] - float(tot)) <= 1e-12 * max(float(tota), 1e-300)
        assert abs(A[e] - float(tota)) <= 1e-12 * max(float(tota), 1e-300)


def test_score_special_cases():
    w = synth.decode_workload("t", 23, [16])
    s = w.signs()
    qc, qs = oracle.quantize(w.q(0, [0])[0], s)
    kc, ks = oracle.quantize(w.keys(0), s)
    _, _, dots = oracle.score_rows(qc, qs, np.zeros(32, np.float32), kc, ks, want_dots=True)
    for j in (0, 7, 31):  # one-hot weights select ReLU of one head
        wt = np.zeros(32, dtype=np.float32)
        wt[j] = 1.0
        I, _ = oracle.score_rows(qc, qs, wt, kc, ks)
        assert np.array_equal(I, np.maximum(dots[j], 0.0))
    # negating every key code flips every dot; then sum of ReLU terms is the sum of the negative parts
    neg_kc = kc ^ np.uint8(0x88)
    ones = np.ones(32, dtype=np.float32)
    I_pos, _ = oracle.score_rows(qc, qs, ones, kc, ks)
    I_neg, _ = oracle.score_rows(qc, qs, ones, neg_kc, ks)
    assert np.allclose(I_pos + I_neg, np.abs(dots).sum(axis=0), rtol=1e-12)
    # all dots negative -> score 0 for any weights
    mask = (dots < 0).all(axis=0)
    q_neg = qc.copy()
    # a query equal to minus a key gives d_j = -|k|^2 < 0 for every head
    kq = np.repeat(kc[3:4] ^ np.uint8(0x88), 32, axis=0)
    kqs = np.repeat(ks[3:4], 32, axis=0)
    I, A = oracle.score_rows(kq, kqs, w.w(0, [0])[0], kc[3:4], ks[3:4])
    assert I[0] == 0.0 and A[0] == 0.0 and math.copysign(1.0, I[0]) == 1.0


def test_mac_count_per_entry_and_pages_totals():
    g = golden("indexer_counts.txt")
    assert g["heads"] * g["head_dim"] == g["macs_per_entry"] == 4096
    w = synth.decode_workload("t", 24, [37])
    s = w.signs()
    qc, qs = oracle.quantize(w.q(0, [0])[0], s)
    kc, ks = oracle.quantize(w.keys(0), s)
    oracle.mac_reset()
    oracle.score_rows(qc, qs, w.w(0, [0])[0], kc, ks)
    per_entry = oracle.mac_count() / 37
    assert per_entry == g["macs_per_entry"]
    # per-token totals at 1M context, from the per-entry count and the visible entry counts
    enc = (1 << 19) * per_entry  # encoder Full layer, m = 2
    dec = (1 << 20) * per_entry  # layer-20 Full and each Reindex layer without the pool, m = 1
    pool = g["pool_blocks"] * g["pool_block_size"]
    assert pool == g["pool_positions_max"] == 16384
    rei = pool * per_entry

    def sig2(x):
        return float(f"{x:.1e}")

    assert sig2(enc) == g["encoder_full_macs_per_layer"]
    assert round((1 << 19) / 1e4) * 1e4 == g["encoder_full_entries_1m"]
    assert round((1 << 20) / 1e4) * 1e4 == g["layer20_entries_1m"]
    assert sig2(dec) == g["layer20_macs"] == g["reindex_macs_no_pool_each"]
    total = 3 * enc + dec + 4 * dec
    assert sig2(total) == g["total_no_pool"]
    assert round(4 * dec / total, 1) == g["reindex_share_no_pool"]
    assert sig2(rei) == g["reindex_macs_with_pool_per_query"]
    assert rei == 67108864
    assert pool / (1 << 20) == g["reindex_fraction_of_1m_scan"]
    assert sig2(4 * dec) == g["reindex_4_layers_no_pool"]
    assert sig2(4 * rei) == g["reindex_4_layers_with_pool"]
    total_pool = 3 * enc + dec + 4 * rei
    assert sig2(total_pool) == g["total_with_pool"]
    assert round(total_pool / total, 1) == g["total_with_pool_fraction"]
    assert pool / g["topk"] == g["pool_over_topk"]
    # format: 128 FP4 codes + one 8-bit scale per group of 32
    assert 4 + 8 / g["group_size_indexer"] == g["bits_per_element_indexer"]
    assert 128 * 4 // 8 + (128 // 32) == g["bytes_per_indexer_entry"]
