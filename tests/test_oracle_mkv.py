"""Pins of the oracle's main-KV codec ([P1] "the scale format decides precision" and "removing
the global scale still leaves enough range"): E4M3 values against PyTorch's float8_e4m3fn
decoder, scale minimality by brute force over every E4M3 value, the pages' byte and range
figures, the tie rule with non-power-of-two scales, round-trip error bounds, and the gather
against an independent numpy decode."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

E2M1_PAGE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # [P1] "E2M1 has only 15 values"


def torch_e4m3(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(b, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def test_e4m3_values_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch_e4m3(b)
    got = np.array([oracle.e4m3_value(int(x)) for x in b])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9 and oracle.e4m3_value(0x38) == 1.0


def test_page_figures():
    # 512 values x 4 bits + one byte per 16 = 256 + 32 = 288 bytes, 4.5 bits per value
    assert oracle.MKV_DIM * 4 // 8 + oracle.MKV_DIM // oracle.MKV_GROUP == 288
    assert 4 + 8 / oracle.MKV_GROUP == 4.5
    # largest representable magnitude 448 x 6 = 2688
    assert oracle.e4m3_value(0x7E) * E2M1_PAGE[-1] == 2688.0
    # neighbouring normal E4M3 values differ by at most 12.5%
    pos = np.array([oracle.e4m3_value(b) for b in range(0x08, 0x7F)])
    assert np.max(pos[1:] / pos[:-1]) <= 1.125 + 1e-15


def test_scale_is_smallest_e4m3_covering_the_group_max():
    finite = np.sort(np.unique(torch_e4m3(np.arange(0, 0x7F, dtype=np.uint8))))
    rng = np.random.default_rng(3)
    samples = np.concatenate([rng.random(500) * 30, 6 * finite[:60], 6 * finite[60:] * (1 + 1e-12), [0.0, 1e-9]])
    for a in samples:
        b = oracle.e4m3_scale_for(a)
        want = finite[np.argmax(6 * finite >= a)] if (6 * finite >= a).any() else 448.0
        assert oracle.e4m3_value(b) == want, a
    assert oracle.e4m3_scale_for(1e6) == 0x7E  # saturates at 448


def bf16_bits(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_ties_to_even_with_non_power_of_two_scale():
    # group max 6 * 1.125 fixes the scale at 1.125 (0x31); midpoints t * 1.125 round to the even code
    s = 1.125
    assert oracle.e4m3_value(oracle.e4m3_scale_for(6 * s)) == s
    mids = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    row = np.zeros(512)
    row[0] = 6 * s
    for i, (t, _) in enumerate(mids.items()):
        row[1 + i] = t * s
        row[8 + i] = -t * s
    x = bf16_bits(row)
    assert np.array_equal(x.view(np.uint16), bf16_bits(row))  # all exactly representable
    codes, scales = oracle.mkv_quantize(x[None, :])
    vals = oracle.mkv_values(codes, scales)[0]
    assert scales[0, 0] == oracle.e4m3_scale_for(6 * s)
    for i, (t, r) in enumerate(mids.items()):
        assert vals[1 + i] == r * s and vals[8 + i] == -r * s, t


def test_rms_normalised_rows_never_saturate_and_round_trip_within_half_a_step():
    rng = np.random.default_rng(7)
    u = rng.standard_normal((40, 512))
    u[:5] *= 1e-3
    u[5:10] = np.where(rng.random((5, 512)) < 0.9, 0.0, u[5:10])  # sparse rows, all-zero groups
    x = u / np.sqrt((u ** 2).mean(axis=1, keepdims=True))  # RMSNorm with unit weights
    x[10, :16] = 0.0
    assert np.abs(x).max() <= math.sqrt(512)  # [P1]: |x_c| <= sqrt(512) ~ 22.6
    xb = bf16_bits(x)
    xv = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    codes, scales = oracle.mkv_quantize(xb)
    vals = oracle.mkv_values(codes, scales)
    s = np.array([[oracle.e4m3_value(b) for b in row] for row in scales]).repeat(16, axis=1)
    g = np.abs(xv).reshape(40, 32, 16).max(axis=2).repeat(16, axis=1)
    assert (s <= 448).all() and (6 * s >= g).all()  # no saturation
    # error at most half the E2M1 gap at that magnitude (gaps 0.5 below 2, 1 up to 4, 2 up to 6)
    gap = np.where(np.abs(xv) <= 2 * s, 0.5, np.where(np.abs(xv) <= 4 * s, 1.0, 2.0)) * s
    assert (np.abs(vals - xv) <= gap / 2 + 1e-300).all()
    assert (vals[10, :16] == 0).all() and (scales[10, 0] == 0)
    # values on the grid survive exactly
    grid = np.array(E2M1_PAGE + [-v for v in E2M1_PAGE[1:]] + [0.0]).repeat(2)[:16] * 0.875
    row = np.tile(grid, 32)
    row[::16] = 6 * 0.875
    c2, s2 = oracle.mkv_quantize(bf16_bits(row)[None, :])
    assert np.array_equal(oracle.mkv_values(c2, s2)[0], row)


def test_gather_matches_numpy_decode_and_is_exact_in_bf16():
    rng = np.random.default_rng(11)
    rows = 300
    codes = rng.integers(0, 256, (rows, 256), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, 32), dtype=np.uint8)  # finite positive scales
    base = np.array([0, 100, 200], dtype=np.int64)
    n = np.array([100, 90, 100], dtype=np.int64)
    idx = np.stack([rng.permutation(100)[:7] for _ in range(3)]).astype(np.int32)
    idx[1, 0] = 95  # past n: zeros
    idx[2, 3] = -1
    out, bad = oracle.mkv_gather(codes, scales, base, n, idx)
    assert bad == 0
    e2m1 = np.array(E2M1_PAGE + [-v for v in E2M1_PAGE])
    e2m1[8] = -0.0
    for t in range(3):
        for i in range(7):
            p = int(idx[t, i])
            if p < 0 or p >= n[t]:
                assert (out[t, i] == 0).all()
                continue
            r = base[t] + p
            nib = np.stack([codes[r] & 15, codes[r] >> 4], axis=1).reshape(-1)
            vals = e2m1[nib] * torch_e4m3(scales[r]).repeat(16)
            assert np.array_equal(out[t, i], bf16_bits(vals)), (t, i)


def test_synthetic_rows_quantise_like_the_definition():
    # the latent rows the benchmarks use: RMS-normalised bf16 rows from the seeded generator
    x = synth.mkv_rows(9, np.array([0, 5, 123456]))
    assert x.shape == (3, 512) and x.dtype == np.uint16
    v = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.abs(np.sqrt((v ** 2).mean(axis=1)) - 1).max() < 0.02
    assert np.array_equal(synth.mkv_rows(9, np.array([123456])), x[2:3])
