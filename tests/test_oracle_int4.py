"""Pins of the oracle's binary16 handling and grouped affine INT4 (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_rounding_matches_numpy():
    gen = np.random.default_rng(1)
    vals = np.concatenate([
        gen.standard_normal(4000) * 10.0 ** gen.integers(-9, 6, 4000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, -1e9,
         2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11,
         1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, -2050.0],
    ])
    for v in vals:
        with np.errstate(over="ignore"):
            want = np.float16(v).view(np.uint16)  # numpy: nearest, ties even
        assert oracle.f16_from_double(float(v)) == int(want), v


def test_int4_hand_made_groups_round_trip():
    """s = 2^-4, z = 8, q cycling 0..15: w = (q - 8) / 16 quantizes back to
    the same codes, scale and zero point; K = 200 has a partial last group."""
    n, k, group = 3, 200, 128
    q_true = (np.arange(n * k).reshape(n, k) + np.arange(n)[:, None]) % 16
    w = ((q_true - 8) * 2.0 ** -4).astype(np.float32)
    q, s, z = oracle.int4_quantize(w, group)
    assert s.shape == (n, 2) and z.shape == (n, 2)
    assert np.all(s == np.float16(2.0 ** -4).view(np.uint16))
    assert np.all(z == np.float16(8.0).view(np.uint16))
    nib = np.empty((n, k), np.int64)
    nib[:, 0::2] = q & 15
    nib[:, 1::2] = q >> 4
    assert np.array_equal(nib, q_true)
    back = oracle.int4_dequantize(q, s, z, n, k, group)
    assert np.array_equal(back, w)


def test_int4_quantizer_error_bound_and_decode_vs_numpy():
    gen = np.random.default_rng(6)
    n, k, group = 40, 328, 128         # last group has 72 elements
    w = (0.02 * gen.standard_normal((n, k))).astype(np.float32)
    w[3, :128] = 0.0                   # an all-zero group
    w[5, 128:256] = np.abs(w[5, 128:256])   # a one-sided group
    q, s, z = oracle.int4_quantize(w, group)
    sv = s.view(np.float16).astype(np.float64)
    zv = z.view(np.float16).astype(np.float64)
    assert np.all(zv == np.round(zv)) and np.all((zv >= 0) & (zv <= 15))
    assert sv[3, 0] == 1.0
    nib = np.empty((n, k), np.int64)
    nib[:, 0::2] = q & 15
    nib[:, 1::2] = q >> 4
    gidx = np.arange(k) // group
    dec = ((nib - zv[:, gidx]) * sv[:, gidx]).astype(np.float32)
    got = oracle.int4_dequantize(q, s, z, n, k, group)
    assert np.array_equal(got, dec)
    # inside the grid span the error is at most half a step; outside it, at
    # most the distance to the span's end
    lo = (0 - zv[:, gidx]) * sv[:, gidx]
    hi = (15 - zv[:, gidx]) * sv[:, gidx]
    wd = w.astype(np.float64)
    err = np.abs(wd - got)
    inside = (wd >= lo) & (wd <= hi)
    assert np.all(err[inside] <= sv[:, gidx][inside] / 2 * (1 + 1e-12))
    outside = ~inside
    dist = np.maximum(lo - wd, wd - hi)
    assert np.all(err[outside] <= dist[outside] + 1e-12)


def test_int4_gemv_one_hot_and_exact():
    gen = np.random.default_rng(8)
    n, k, group = 8, 200, 128
    w = (0.02 * gen.standard_normal((n, k))).astype(np.float32)
    q, s, z = oracle.int4_quantize(w, group)
    deq = oracle.int4_dequantize(q, s, z, n, k, group)
    for j in (0, 127, 128, 199):
        x = np.zeros(k, np.uint16)
        x[j] = 0x3F80
        y, _ = oracle.int4_gemv(q, s, z, n, k, group, x)
        assert np.array_equal(y[0], deq[:, j].astype(np.float64))
    x = workloads.random_bits_bf16(gen, (k,), -6, 6)
    y, S = oracle.int4_gemv(q, s, z, n, k, group, x)
    xf = workloads.bf16_to_f32(x)
    for r in range(n):
        exact = sum(Fraction(float(deq[r, j])) * Fraction(float(xf[j])) for j in range(k))
        assert abs(Fraction(y[0, r]) - exact) <= Fraction((k + 2) * 2.0 ** -53 * S[0, r])


def test_int4_scale_overflow_is_reported():
    w = np.array([[-1e6, 1e6]], np.float32)
    with pytest.raises(OverflowError):
        oracle.int4_quantize(w, 128)
