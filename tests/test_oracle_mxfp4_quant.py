"""Pins of the CPU oracle's MXFP4 quantizer and row-postscale fit (no GPU).

The quantizer is pinned by hand-worked blocks of the OCP MX conversion rule
(tests/golden/mxfp4_quantize_blocks.txt), by an exact round trip through
the oracle's own decode of blocks whose scale the rule must reproduce, by a
brute-force nearest-value check over all 16 codes, and by the rule's error
bound.  The postscale fit is pinned by numpy's least-squares solver and by
the properties of a least-squares fit.
"""
import numpy as np
import pytest

import oracle
from _golden import lines

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def unpack_codes(codes, k):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (k,), np.int64)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def golden_cases():
    cases, cur = [], None
    for t in lines("mxfp4_quantize_blocks.txt"):
        if t[0] == "case":
            cur = dict(name=t[1], vals={}, codes={})
            cases.append(cur)
        elif t[0] == "k":
            cur["k"] = int(t[1])
        elif t[0] == "vals":
            cur["vals"].update({i: float(v) for i, v in enumerate(t[1:])})
        elif t[0] == "set":
            cur["vals"][int(t[1])] = float(t[2])
        elif t[0] == "scales":
            cur["scales"] = [int(v) for v in t[1:]]
        elif t[0] == "codes":
            cur["codes"].update({i: int(v) for i, v in enumerate(t[1:])})
        elif t[0] == "code":
            cur["codes"][int(t[1])] = int(t[2])
    return cases


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_quantize_hand_worked_blocks(case):
    k = case["k"]
    w = np.zeros((1, k), np.float32)
    for i, v in case["vals"].items():
        w[0, i] = v
    codes, scales, _ = oracle.mxfp4_quantize(w, fit_postscale=False)
    want = np.zeros(k, np.int64)
    for i, c in case["codes"].items():
        want[i] = c
    assert scales[0].tolist() == case["scales"]
    assert unpack_codes(codes, k)[0].tolist() == want.tolist()


def test_round_trip_through_decode_is_exact():
    """Blocks whose largest magnitude is a code of value 4 or 6 decode to
    values from which the rule must recover the same scale and codes
    (including -0)."""
    gen = np.random.default_rng(7)
    n, k = 48, 256
    c = gen.integers(0, 16, (n, k))
    blocks = c.reshape(n, k // 32, 32)
    pos = gen.integers(0, 32, (n, k // 32))
    big = gen.choice([6, 7, 14, 15], (n, k // 32))
    np.put_along_axis(blocks, pos[..., None], big[..., None], axis=2)
    c = blocks.reshape(n, k)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    scales = gen.integers(2, 250, (n, k // 32)).astype(np.uint8)
    w = oracle.mxfp4_dequantize(packed, scales, n, k)
    codes2, scales2, ps = oracle.mxfp4_quantize(w)
    assert np.array_equal(scales2, scales)
    assert np.array_equal(codes2, packed)
    assert np.all(ps == 1.0)   # the decoded row is reproduced exactly


def _decode_exact(codes, scales, k):
    c = unpack_codes(codes, k)
    mag = GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1)
    return mag * np.exp2(e.astype(np.float64))


def test_nearest_code_brute_force_and_error_bound():
    gen = np.random.default_rng(8)
    n, k = 64, 512
    w = (gen.standard_normal((n, k)) *
         np.exp2(gen.integers(-12, 12, (n, 1)))).astype(np.float32)
    w[3, :40] = 0.0
    codes, scales, _ = oracle.mxfp4_quantize(w, fit_postscale=False)
    d = _decode_exact(codes, scales, k)
    X = np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=-1).astype(np.float64))
    v = w.astype(np.float64) / X
    # every element's code is the nearest of the 8 magnitudes (sign kept),
    # ties to the even index, magnitudes >= 6 on 6
    dist = np.abs(np.abs(v)[..., None] - GRID)
    best = dist.min(axis=-1)
    got = np.abs(d / X)
    assert np.all(np.abs(np.abs(got) - np.abs(v)) == best)
    # error bound of the rule: half the grid spacing below 6, clamp above
    a = np.abs(v)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.where(a <= 6, half, a - 6)
    assert np.all(np.abs(v - d / X) <= bound)
    # the scale puts every block's largest magnitude in [4, 8)
    amax = np.abs(v).reshape(n, k // 32, 32).max(axis=-1)
    nz = amax > 0
    assert np.all((amax[nz] >= 4) & (amax[nz] < 8))


def test_postscale_is_the_least_squares_fit():
    gen = np.random.default_rng(9)
    n, k = 40, 384
    w = (0.02 * gen.standard_normal((n, k))).astype(np.float32)
    codes, scales, ps = oracle.mxfp4_quantize(w)
    d = _decode_exact(codes, scales, k)
    wd = w.astype(np.float64)
    for r in range(n):
        sol = np.linalg.lstsq(d[r][:, None], wd[r], rcond=None)[0][0]
        assert abs(float(ps[r]) - sol) <= 2 * np.spacing(np.float32(sol)), r
        res = wd[r] - float(ps[r]) * d[r]
        # residual orthogonal to the decoded row, error never above ps = 1
        assert abs(res @ d[r]) <= 1e-6 * np.linalg.norm(wd[r]) * np.linalg.norm(d[r])
        assert res @ res <= (wd[r] - d[r]) @ (wd[r] - d[r]) * (1 + 1e-9)


def test_postscale_of_zero_row_is_one_and_nonfinite_is_rejected():
    w = np.zeros((2, 64), np.float32)
    w[1, 5] = 3.0
    _, scales, ps = oracle.mxfp4_quantize(w)
    assert ps[0] == 1.0 and ps[1] == 1.0
    assert scales[0].tolist() == [0, 0]
    for bad in (np.inf, -np.inf, np.nan):
        w2 = w.copy()
        w2[1, 7] = bad
        with pytest.raises(ValueError):
            oracle.mxfp4_quantize(w2)
