"""Seeded input generator: determinism, random access, recipe properties (CPU only)."""
from fractions import Fraction

import numpy as np

import synth


def test_deterministic_and_random_access():
    a = synth.normal_bf16(9, 3, 2, 0, 5000)
    b = synth.normal_bf16(9, 3, 2, 0, 5000)
    assert np.array_equal(a, b)
    assert np.array_equal(synth.normal_bf16(9, 3, 2, 1234, 100), a[1234:1334])
    assert not np.array_equal(synth.normal_bf16(9, 3, 3, 0, 100), a[:100])
    x = synth.bf16_to_f64(synth.normal_bf16(9, 2, 0, 0, 200000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_bf16_rounding_nearest_even():
    for v in [1.0, 1.00390625, 1.005859375, 1.0078125, -3.1415926, 1e-3, 123456.7]:
        h = synth.bf16_rne(v)
        got = synth.bf16_to_f64(np.array([h], np.uint16))[0]
        # neighbours on the bf16 grid around v
        e = Fraction(2) ** (int(np.floor(np.log2(abs(v)))) - 7)
        lo = (Fraction(v) / e).__floor__() * e
        cands = [lo, lo + e]
        best = min(cands, key=lambda c: (abs(c - Fraction(v)), (c / e) % 2))
        assert Fraction(got) == best


def test_workload_keys_slices_and_planting():
    w = synth.decode_workload("t", 5, [3000, 1000])
    full = w.keys(0)
    assert np.array_equal(w.keys(0, 100, 50), full[100:150])
    pos = w.planted(0)
    assert len(pos) == 30 and len(set(pos.tolist())) == 30 and pos.min() >= 0 and pos.max() < 3000
    assert np.array_equal(w.key_rows(0, pos[:3]), full[pos[:3]])
    raw = synth.normal_bf16(5, synth.TAG_K, 0, 0, 3000 * 128).reshape(3000, 128)
    changed = np.where((raw != full).any(axis=1))[0]
    assert set(changed.tolist()) <= set(pos.tolist())


def test_configs_shapes():
    c2 = synth.config("decode_batch64")
    assert c2.nq == 64 and (c2.seq_len >= 65536).all() and (c2.seq_len <= 131072).all()
    c5 = synth.config("prefill_128k")
    assert c5.nq == 4096 and c5.n_vis[0] == 126977 and c5.n_vis[-1] == 131072
    c4 = synth.config("fullscan_1m")
    assert c4.nq == 8 and (c4.n_vis == 1 << 20).all()
    assert c5.group == 4096 and c4.group == 1


def test_spec_decode_shape():
    # the token plus 5 draft positions per sequence: 6 consecutive queries sharing the sequence's
    # keys, position j of a sequence of n entries seeing n - 5 + j of them
    w = synth.config("spec_decode_1m")
    assert w.nseq == 8 and w.nq == 48 and w.group == 6 and w.layers == 4
    assert np.array_equal(w.qseq, np.repeat(np.arange(8), 6))
    assert np.array_equal(w.n_vis[:6], (1 << 20) - 5 + np.arange(6))
    assert (w.k_base[6:12] == 1 << 20).all() and (w.k_base[:6] == 0).all()
    assert np.array_equal(w.plant_query, np.arange(8) * 6)


def test_token_schedule_shape_and_page_total():
    # 3 encoder Full layers (own caches, m = 2) + decoder Full + 4 Reindex layers over the pool:
    # 3 x 2^19 x 4096 + 2^20 x 4096 + 4 x 16384 x 4096 MACs per token = 1.1e10 (the page's total)
    encs, dec = synth.token_1m()
    assert len(encs) == 3 and all(w.nq == 8 and (w.n_vis == 1 << 19).all() for w in encs)
    assert len({w.seed for w in encs}) == 3 and dec.layers == 4 and (dec.n_vis == 1 << 20).all()
    macs = (sum(int(w.n_vis[0]) for w in encs) + int(dec.n_vis[0]) + dec.layers * 16384) * 4096
    assert float(f"{macs:.1e}") == 1.1e10
