"""Pins of the CPU oracle's MXFP4 decode and matvec (no GPU).

Each check ties the oracle to something other than itself: the OCP E2M1
value table, exact rational arithmetic, integer matmul in numpy, or exact
algebraic invariants.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from _golden import e2m1_table, lines

U64 = 2.0 ** -53


def gamma(n):
    return n * U64 / (1 - n * U64)


def f32_bits(v):
    return np.array([v], dtype=np.float32).view(np.uint32)[0]


def test_e2m1_values_match_ocp_table():
    table = e2m1_table()
    assert sorted(table) == list(range(16))
    for code, v in table.items():
        got = oracle.e2m1_value(code)
        assert got == v
        assert math.copysign(1.0, got) == math.copysign(1.0, v), code


def test_decode_every_code_times_every_scale():
    """16 codes x 256 scale bytes, bit-exact against the exact rational
    value rounded once to fp32 (numpy's rounding)."""
    table = e2m1_table()
    for e in range(256):
        for code in range(16):
            got = oracle.mxfp4_weight(code, e)
            if e == 255:
                assert np.isnan(got)
                continue
            exact = Fraction(table[code]) * Fraction(2) ** (e - 127)
            with np.errstate(over="ignore"):
                want = np.float32(float(exact))
            if table[code] == 0.0 and math.copysign(1.0, table[code]) < 0:
                want = np.float32(-0.0)
            assert f32_bits(got) == f32_bits(want), (code, e, got, want)


def test_decode_edge_semantics():
    # E8M0 byte 0 is 2^-127 (an fp32 subnormal), not zero.
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.mxfp4_weight(1, 0) == np.float32(2.0 ** -128)
    # Overflow to infinity once the product leaves fp32.
    assert np.isinf(oracle.mxfp4_weight(7, 254))
    assert oracle.mxfp4_weight(3, 254) == np.float32(1.5 * 2.0 ** 127)
    # NaN scale poisons the block.
    assert np.isnan(oracle.mxfp4_weight(0, 255))
    # Code 8 is negative zero.
    assert f32_bits(oracle.mxfp4_weight(8, 127)) == 0x80000000


def test_nibble_order_golden():
    rows = {r[0]: r[1:] for r in lines("mxfp4_nibble_order.txt") if r[0] != "elem"}
    elems = [(int(a), float(b)) for t, a, b in
             (r for r in lines("mxfp4_nibble_order.txt") if r[0] == "elem")]
    codes = np.array([int(b, 16) for b in rows["codes"]], np.uint8).reshape(1, 32)
    scales = np.array([int(b) for b in rows["scales"]], np.uint8).reshape(1, 2)
    w = oracle.mxfp4_dequantize(codes, scales, 1, 64)
    for k, v in elems:
        assert w[0, k] == v, (k, w[0, k], v)


def _exact_gemv(codes, scales, ps, x_bits, n, k):
    """Exact rational y and S of the same definition, from the OCP table."""
    table = e2m1_table()
    xs = [Fraction(float(v)) for v in workloads.bf16_to_f32(x_bits)]
    ys, Ss = [], []
    for r in range(n):
        acc, mag = Fraction(0), Fraction(0)
        for j in range(k):
            byte = int(codes[r, j // 2])
            c = byte >> 4 if j & 1 else byte & 15
            wv = Fraction(table[c]) * Fraction(2) ** (int(scales[r, j // 32]) - 127)
            t = wv * xs[j]
            acc += t
            mag += abs(t)
        p = Fraction(float(ps[r]))
        ys.append(p * acc)
        Ss.append(abs(p) * mag)
    return ys, Ss


@pytest.mark.parametrize("elo,ehi", [(119, 125), (2, 252), (100, 150)])
def test_gemv_bruteforce_4x32_exact_rational(elo, ehi):
    gen = np.random.default_rng([7, elo, ehi])
    for trial in range(6):
        n, k = 4, 32 * (1 + trial % 2)
        codes = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
        scales = gen.integers(elo, ehi + 1, (n, k // 32), dtype=np.uint8)
        ps = gen.uniform(0.25, 4.0, n).astype(np.float32)
        x = workloads.random_bits_bf16(gen, (k,), -10, 10)
        y, S = oracle.mxfp4_gemv(codes, scales, ps, n, k, x)
        ey, eS = _exact_gemv(codes, scales, ps, x, n, k)
        for r in range(n):
            bound = gamma(k + 2) * float(eS[r])
            assert abs(Fraction(y[0, r]) - ey[r]) <= Fraction(bound), (trial, r)
            assert abs(S[0, r] - float(eS[r])) <= gamma(k + 2) * float(eS[r])


def test_gemv_reduces_to_integer_matmul():
    """Scale byte 127 and postscale 1: weights are halves of integers, x are
    small integers, so y equals an int64 matmul exactly."""
    table = e2m1_table()
    gen = np.random.default_rng(11)
    n, k = 24, 256
    codes = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = np.full((n, k // 32), 127, np.uint8)
    xi = gen.integers(-8, 9, k)
    x = workloads.bf16_bits(xi.astype(np.float32))
    y, _ = oracle.mxfp4_gemv(codes, scales, None, n, k, x)
    nib = np.empty((n, k), np.int64)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    w2 = np.vectorize(lambda c: int(2 * table[int(c)]))(nib).astype(np.int64)
    want = (w2 @ xi.astype(np.int64)) / 2.0
    assert np.array_equal(y[0], want)


def test_gemv_exact_invariants():
    gen = np.random.default_rng(5)
    n, k = 32, 512
    codes = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = gen.integers(119, 126, (n, k // 32), dtype=np.uint8)
    ps = gen.uniform(0.5, 1.5, n).astype(np.float32)
    x = workloads.bf16_bits(gen.standard_normal(k).astype(np.float32))
    y, _ = oracle.mxfp4_gemv(codes, scales, ps, n, k, x)
    # every block scale doubled -> exactly doubled
    y2, _ = oracle.mxfp4_gemv(codes, scales + 1, ps, n, k, x)
    assert np.array_equal(y2, 2 * y)
    # postscale doubled -> exactly doubled
    y3, _ = oracle.mxfp4_gemv(codes, scales, 2 * ps, n, k, x)
    assert np.array_equal(y3, 2 * y)
    # row permutation -> permuted outputs
    perm = gen.permutation(n)
    y4, _ = oracle.mxfp4_gemv(codes[perm], scales[perm], ps[perm], n, k, x)
    assert np.array_equal(y4[0], y[0, perm])
    # selected rows equal the full result
    y5, _ = oracle.mxfp4_gemv(codes, scales, ps, n, k, x, rows=[3, 17, 30])
    assert np.array_equal(y5[0], y[0, [3, 17, 30]])
    # a batch of two tokens equals two single calls
    xb = np.stack([x, x[::-1]])
    yb, _ = oracle.mxfp4_gemv(codes, scales, ps, n, k, xb)
    yr, _ = oracle.mxfp4_gemv(codes, scales, ps, n, k, x[::-1].copy())
    assert np.array_equal(yb[0], y[0]) and np.array_equal(yb[1], yr[0])


def test_gemv_one_hot_column():
    """x = e_j gives ps_r * w[r, j] as one exactly rounded product."""
    table = e2m1_table()
    gen = np.random.default_rng(3)
    n, k = 16, 64
    codes = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = gen.integers(2, 253, (n, k // 32), dtype=np.uint8)
    ps = gen.uniform(0.5, 1.5, n).astype(np.float32)
    for j in (0, 1, 31, 32, 63):
        x = np.zeros(k, np.uint16)
        x[j] = 0x3F80          # 1.0
        y, _ = oracle.mxfp4_gemv(codes, scales, ps, n, k, x)
        for r in range(n):
            b = int(codes[r, j // 2])
            c = b >> 4 if j & 1 else b & 15
            wv = Fraction(table[c]) * Fraction(2) ** (int(scales[r, j // 32]) - 127)
            assert Fraction(y[0, r]) == wv * Fraction(float(ps[r]))
