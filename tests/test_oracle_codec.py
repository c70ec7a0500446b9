"""Pins for the oracle's rotation and MXFP4 encoder (CPU only).

Each check ties the oracle to something other than itself: the value set printed on the pages,
a textbook round-to-nearest-even written with a different algorithm, scipy's Hadamard matrix,
orthogonality, and exact rational arithmetic.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_e2m1():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        lines = [l for l in f if l.strip() and not l.startswith("#")]
    return [float(v) for v in lines[0].split()]


def test_e2m1_value_set_matches_pages():
    mags = golden_e2m1()
    assert len(mags) == 8
    vals = {oracle.e2m1_value(c) for c in range(16)}
    expect = set(mags) | {-m for m in mags}
    assert vals == expect
    assert len(vals) == 15  # "15 values": +0 and -0 coincide
    # codes 0..7 are the magnitudes in ascending order, bit 3 is the sign
    assert [oracle.e2m1_value(c) for c in range(8)] == mags
    assert [oracle.e2m1_value(c | 8) for c in range(1, 8)] == [-m for m in mags[1:]]


def textbook_rne_e2m1(v: float) -> float:
    """Round to the E2M1 grid with IEEE nearest-even: spacing 0.5 below 2, 1 below 4, 2 above."""
    a = abs(v)
    spacing = 0.5 if a < 2 else (1.0 if a < 4 else 2.0)
    q = float(np.rint(a / spacing)) * spacing
    return math.copysign(q, v) if q != 0 else 0.0


def test_e2m1_rounding_against_textbook_rne():
    grid = np.arange(-6 * 256, 6 * 256 + 1) / 256.0  # every multiple of 1/256 in [-6, 6]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10)])
    vals = np.concatenate([grid, near, -near])
    for v in vals:
        code = oracle.e2m1_code(float(v))
        got = oracle.e2m1_value(code)
        assert got == textbook_rne_e2m1(float(v)), (v, code, got)
        if got == 0.0:
            assert code == 0, "a value that rounds to zero is +0"


def test_e2m1_tie_directions():
    # ties go to the even mantissa bit: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    expect = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, q in expect.items():
        assert oracle.e2m1_value(oracle.e2m1_code(v)) == q
        assert oracle.e2m1_value(oracle.e2m1_code(-v)) == -q if q else True


def exact_scale_exp(a: float) -> int:
    """smallest e with 6 * 2^e >= a, by exact rational search from a bit-length estimate."""
    if a == 0:
        return -127
    fa = Fraction(a)
    e = (fa.numerator.bit_length() - fa.denominator.bit_length()) - 4
    while Fraction(6) * Fraction(2) ** e < fa:
        e += 1
    return max(-127, min(127, e))


def test_scale_exp_known_values():
    assert oracle.scale_exp(6.0) == 0
    assert oracle.scale_exp(float(np.nextafter(np.float32(6.0), np.float32(7.0)))) == 1
    assert oracle.scale_exp(3.0) == -1
    assert oracle.scale_exp(float(np.nextafter(np.float32(3.0), np.float32(4.0)))) == 0
    assert oracle.scale_exp(0.0) == -127
    assert oracle.scale_exp(1e-45) == -127  # clamped at the bottom of UE8M0


def test_scale_exp_against_exact_rational():
    rng = np.random.default_rng(7)
    vals = np.concatenate([np.abs(rng.standard_normal(3000)).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 3000),
                           (6.0 * 2.0 ** np.arange(-60, 60)).astype(np.float32)])
    for a in vals.astype(np.float64):
        e = oracle.scale_exp(float(a))
        assert e == exact_scale_exp(float(a))
        if a > 0 and -127 < e:
            assert 6.0 * 2.0 ** e >= a > 6.0 * 2.0 ** (e - 1)


def test_quantize_roundtrip_every_grid_value_every_scale():
    mags = golden_e2m1()
    signed = [m for m in mags] + [-m for m in mags[1:]]
    for e in range(-20, 21):
        row = np.zeros(128, dtype=np.float64)
        for g in range(4):
            grp = [signed[(g * 7 + c) % len(signed)] for c in range(32)]
            grp[5] = 6.0  # forces the scale exponent to exactly e
            row[g * 32:(g + 1) * 32] = np.array(grp) * 2.0 ** e
        codes, scales = oracle.quantize_rotated(row.astype(np.float32))
        assert (scales[0] == e + 127).all()
        for i in range(128):
            c = (codes[0, i // 2] >> (4 * (i & 1))) & 15
            assert oracle.e2m1_value(int(c)) * 2.0 ** e == row[i]
            if row[i] == 0:
                assert c == 0


def test_quantize_nibble_order():
    row = np.zeros(128, dtype=np.float32)
    row[0], row[1] = 6.0, 0.5  # element 0 -> low nibble, element 1 -> high nibble of byte 0
    codes, scales = oracle.quantize_rotated(row)
    assert codes[0, 0] == (7 | (1 << 4))
    assert scales[0, 0] == 127


def test_max_element_lands_on_top_codes():
    # with e rounded up, max|y| / 2^e lies in (3, 6], so the largest element codes to 3, 4 or 6
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((200, 128)) * 10.0 ** rng.uniform(-3, 3, (200, 1))).astype(np.float32)
    codes, scales = oracle.quantize_rotated(y)
    for r in range(200):
        for g in range(4):
            grp = y[r, g * 32:(g + 1) * 32]
            i = g * 32 + int(np.argmax(np.abs(grp)))
            c = (codes[r, i // 2] >> (4 * (i & 1))) & 7
            assert abs(oracle.e2m1_value(int(c))) in (3.0, 4.0, 6.0)


def test_inv_sqrt128_constant():
    assert oracle.inv_sqrt128_f32() == float(np.float32(2.0 ** -3.5))


def test_rotation_against_scipy_hadamard():
    H = scipy.linalg.hadamard(128).astype(np.float64)
    s = synth.signs(11)
    x = synth.normal_bf16(11, 3, 0, 0, 128 * 64).reshape(64, 128)
    xf = synth.bf16_to_f64(x)
    S = (H @ (s[None, :].astype(np.float64) * xf).T).T  # exact: bf16 inputs, 128 terms, fp64
    expect = (S.astype(np.float32) * np.float32(2.0 ** -3.5)).astype(np.float32)
    got = oracle.rotate(x, s)
    assert np.array_equal(got, expect)


def test_rotation_is_orthonormal():
    s = np.ones(128, dtype=np.int8)
    x = synth.normal_bf16(12, 3, 0, 0, 128 * 32).reshape(32, 128)
    xf = synth.bf16_to_f64(x)
    y = oracle.rotate(x, s).astype(np.float64)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(xf, axis=1), rtol=1e-6)
    # H/sqrt(128) is symmetric and orthogonal: applying it twice returns the input
    y_bf = np.array([[synth.bf16_rne(v) for v in row] for row in y[:4]], dtype=np.uint16)
    z = oracle.rotate(y_bf, s).astype(np.float64)
    assert np.allclose(z, xf[:4], atol=0.05)


def test_rotation_preserves_q_dot_k():
    s = synth.signs(13)
    q = synth.normal_bf16(13, 2, 0, 0, 128 * 16).reshape(16, 128)
    k = synth.normal_bf16(13, 3, 0, 0, 128 * 16).reshape(16, 128)
    dq, dk = oracle.rotate(q, s).astype(np.float64), oracle.rotate(k, s).astype(np.float64)
    ref = synth.bf16_to_f64(q) @ synth.bf16_to_f64(k).T
    assert np.allclose(dq @ dk.T, ref, atol=1e-4)


def test_quantize_rows_equals_rotate_then_quantize():
    s = synth.signs(14)
    x = synth.normal_bf16(14, 3, 0, 0, 128 * 300).reshape(300, 128)
    c1, s1 = oracle.quantize(x, s, nthreads=4)
    c2, s2 = oracle.quantize_rotated(oracle.rotate(x, s))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_dequantised_error_is_bounded():
    # |x - x_hat| <= half a grid step; the step is at most 2 * 2^e (between 4 and 6)
    s = synth.signs(15)
    x = synth.normal_bf16(15, 3, 0, 0, 128 * 50).reshape(50, 128)
    y = oracle.rotate(x, s).astype(np.float64)
    codes, scales = oracle.quantize_rotated(y.astype(np.float32))
    for r in range(50):
        for i in range(128):
            c = (codes[r, i // 2] >> (4 * (i & 1))) & 15
            e = int(scales[r, i // 32]) - 127
            xh = oracle.e2m1_value(int(c)) * 2.0 ** e
            assert abs(xh - y[r, i]) <= 1.0 * 2.0 ** e + 1e-30
