"""Pins of the CPU oracle's FP8 E4M3 decode and row-scaled matvec (no GPU).

The decode is pinned by hand-worked values of the OCP E4M3 definition and
by torch's own float8_e4m3fn conversion of all 256 codes; the matvec by
exact rational brute force, an integer special case that numpy's integer
matmul computes exactly, and exact scaling invariants.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from _golden import lines

U64 = 2.0 ** -53


def test_fp8_values_hand_worked():
    for code, v in lines("ocp_fp8_e4m3_values.txt"):
        got = oracle.fp8e4m3_value(int(code, 16))
        want = float(v)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_fp8_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.fp8e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _finite_codes(gen, shape):
    c = gen.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def test_fp8_gemv_exact_rational_brute_force():
    gen = np.random.default_rng(3)
    n, k, batch = 4, 48, 2
    w = _finite_codes(gen, (n, k))
    scale = gen.uniform(0.5, 2.0, n).astype(np.float32)
    x = workloads.bf16_bits(gen.standard_normal((batch, k)).astype(np.float32))
    y, S = oracle.fp8_gemv(w, scale, n, k, x)
    xv = workloads.bf16_to_f32(x)
    for b in range(batch):
        for r in range(n):
            acc = sum(Fraction(oracle.fp8e4m3_value(int(w[r, j]))) * Fraction(float(xv[b, j]))
                      for j in range(k))
            exact = Fraction(float(scale[r])) * acc
            bound = (k + 2) * U64 / (1 - (k + 2) * U64) * S[b, r]
            assert abs(Fraction(y[b, r]) - exact) <= Fraction(bound), (b, r)


def test_fp8_gemv_integer_case_and_scaling_invariants():
    gen = np.random.default_rng(4)
    n, k = 16, 160
    # codes of the integers 1..15 and their negatives (exact in E4M3)
    ints = np.arange(1, 16)
    table = {int(round(oracle.fp8e4m3_value(c))): c for c in range(0x38, 0x58)
             if float(oracle.fp8e4m3_value(c)).is_integer()}
    vals = gen.choice(ints, (n, k)) * gen.choice([-1, 1], (n, k))
    w = np.array([[table[abs(v)] | (0x80 if v < 0 else 0) for v in row] for row in vals],
                 np.uint8)
    xi = gen.integers(-8, 9, (3, k))
    x = workloads.bf16_bits(xi.astype(np.float32))
    y1, _ = oracle.fp8_gemv(w, None, n, k, x)
    assert np.array_equal(y1, (xi @ vals.T).astype(np.float64))
    # power-of-two and negated scales act exactly on the full-row sum
    for s in (2.0 ** -7, 8.0, -0.5):
        ys, _ = oracle.fp8_gemv(w, np.full(n, s, np.float32), n, k, x)
        assert np.array_equal(ys, s * y1)
    # fp32 activations with the same values give the same result
    yf, _ = oracle.fp8_gemv(w, None, n, k, xi.astype(np.float32))
    assert np.array_equal(yf, y1)
    # selected rows
    rows = np.array([0, 7, 15])
    yr, _ = oracle.fp8_gemv(w, None, n, k, x, rows=rows)
    assert np.array_equal(yr, y1[:, rows])
