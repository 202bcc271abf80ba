"""Pins of the oracle's K/V quantiser and its fp16 rounding (CPU only).

The pages give int8 codes with one fp16 scale per 64 dims but no rounding
rule; the oracle takes the plain absmax reading (scale = fp16(absmax / 127),
code = clamp(rint(x / scale), -127, 127), decided in IEEE fp32).  Each test
below checks the oracle against something other than its own arithmetic:
numpy's float16 conversion, inputs built on an exact grid whose codes and
scales are known in advance, exact rational rounding, and symmetry and error
bounds that any correct absmax quantiser satisfies.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(11)
    parts = [
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 5, 20000),
        # exact midpoints between neighbouring fp16 values (ties to even)
        (np.arange(-3000, 3000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10),
        (np.arange(1, 3000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1e-30], dtype=np.float32),
    ]
    x = np.concatenate(parts)
    got = oracle.f32_to_f16(x).view(np.uint16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def _grid_rows(rng, rows, D=256, block=64):
    """Rows whose every block is code * s for a known fp16 scale s (a small
    odd mantissa times a power of two) and codes with |code| = 127 present,
    so that absmax / 127 == s exactly and x / s == code exactly."""
    nb = D // block
    codes = rng.integers(-127, 128, (rows, D)).astype(np.int64)
    for r in range(rows):
        for b in range(nb):
            codes[r, b * block + rng.integers(block)] = 127 * rng.choice([-1, 1])
    mant = rng.choice([1, 3, 5, 7, 9, 11, 13, 15], (rows, nb))
    expo = rng.integers(-20, 0, (rows, nb))
    s = mant * np.power(2.0, expo)
    x = codes * np.repeat(s, block, axis=1)
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)  # exact in fp16
    return x.astype(np.float16), codes.astype(np.int8), s.astype(np.float16)


def test_quantize_recovers_an_exact_grid():
    rng = np.random.default_rng(5)
    x, codes, s = _grid_rows(rng, 40)
    got_c, got_s = oracle.quantize(x)
    assert np.array_equal(got_s.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(got_c, codes)


def test_quantize_zero_and_vanishing_blocks():
    x = np.zeros((2, 256), dtype=np.float16)
    x[1, 64] = np.float16(2.0 ** -24)     # absmax / 127 rounds to fp16 zero
    x[1, 130] = np.float16(-2.0 ** -24)
    c, s = oracle.quantize(x)
    assert not c.any()
    assert not s.view(np.uint16).any()


def test_quantize_ties_go_to_even_codes():
    # every block holds 127 (scale 1) and 63 values k + 1/2, exact in fp16,
    # whose quotient by the scale is an exact tie
    k = np.arange(-126, 126).reshape(4, 63)
    x = np.zeros((1, 4, 64), dtype=np.float64)
    x[0, :, 0] = 127.0
    x[0, :, 1:] = k + 0.5
    c, s = oracle.quantize(x.reshape(1, 256).astype(np.float16))
    assert np.all(s.astype(np.float64) == 1.0)
    want = np.where(k % 2 == 0, k, k + 1)           # the even neighbour of k + 1/2
    assert np.array_equal(c.reshape(4, 64)[:, 1:].astype(np.int64), want)


def test_quantize_sign_symmetry_and_error_bound():
    rng = np.random.default_rng(7)
    mag = np.float32(10.0) ** rng.integers(-6, 4, (64, 4, 1))
    x = (rng.standard_normal((64, 4, 64)) * mag).reshape(64, 256).astype(np.float16)
    c, s = oracle.quantize(x)
    cn, sn = oracle.quantize(-x)
    assert np.array_equal(cn.astype(np.int64), -c.astype(np.int64))
    assert np.array_equal(sn.view(np.uint16), s.view(np.uint16))
    xs = x.astype(np.float64)
    ss = np.repeat(s.astype(np.float64), 64, axis=1)
    amax = np.repeat(np.abs(xs).reshape(64, 4, 64).max(axis=2), 64, axis=1)
    err = np.abs(xs - c.astype(np.float64) * ss)
    # blocks whose scale is a normal fp16 (>= 2^-14): relative error of the
    # scale <= 2^-11, so only the largest magnitudes can need clamping
    normal = ss >= 2.0 ** -14
    inner = (np.abs(c) < 127) & normal
    clamped = (np.abs(c) == 127) & normal
    assert normal.mean() > 0.5
    assert np.all(err[inner] <= 0.5 * ss[inner] * (1 + 2.0 ** -10))
    assert np.all(np.abs(xs[clamped]) >= 126.5 * ss[clamped] * (1 - 2.0 ** -10))
    assert np.all(np.abs(c) <= 127)
    # a zero scale (absmax / 127 below half the smallest fp16) zeroes the block
    assert not c[ss == 0].any()
    # the scale is the fp16 value nearest absmax / 127
    ref = (amax[:, ::64] / 127.0).astype(np.float16)
    assert np.array_equal(s.view(np.uint16), ref.view(np.uint16))


def test_quantize_codes_are_exact_rational_rounding():
    # nearest integer to the exact quotient x / scale, ties to even, clamped;
    # quotients within 2^-14 of a half-integer are skipped (there the fp32
    # division may round onto the tie)
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((6, 256)) * 3).astype(np.float16)
    c, s = oracle.quantize(x)
    checked = 0
    for r in range(x.shape[0]):
        for d in range(256):
            sc = Fraction(float(s[r, d // 64]))
            q = Fraction(float(x[r, d])) / sc
            fl = q.numerator // q.denominator
            frac = q - fl
            if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 14):
                continue
            n = fl + (1 if frac > Fraction(1, 2) else 0)
            n = max(-127, min(127, n))
            assert int(c[r, d]) == n, (r, d)
            checked += 1
    assert checked > 1500


@pytest.mark.parametrize("rows", [0, 1, 3])
def test_quantize_shapes(rows):
    x = np.ones((rows, 256), dtype=np.float16)
    c, s = oracle.quantize(x)
    assert c.shape == (rows, 256) and s.shape == (rows, 4)
    if rows:
        assert np.all(c == 127) and np.all(s == np.float16(1 / 127))
