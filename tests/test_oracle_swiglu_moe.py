"""Pins of the oracle's activation, gate/up fusion, routing and expert
combine (no GPU)."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4
    assert abs(oracle.silu(math.log(3.0)) - 0.75 * math.log(3.0)) <= 4e-16
    # sigmoid(-ln 3) = 1/4
    assert abs(oracle.silu(-math.log(3.0)) + 0.25 * math.log(3.0)) <= 4e-16
    # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    for z in np.linspace(-30, 30, 241):
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) <= 4e-16 * max(1.0, abs(z))
    # saturation
    assert oracle.silu(800.0) == 800.0
    assert oracle.silu(-800.0) == 0.0


def _one_hot(k, j):
    x = np.zeros(k, np.uint16)
    x[j] = 0x3F80
    return x


def test_gateup_applies_silu_to_gate_only():
    """With x = e_j both projections are single exact products, so h must be
    silu(g) * u with silu on the gate side -- swapping the roles is caught."""
    w = workloads.TINY
    g, u = workloads.gateup(w)
    for j in (0, 77, 255):
        out = oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, _one_hot(w.hidden, j))
        gy, _ = oracle.mxfp4_gemv(*g, w.inter, w.hidden, _one_hot(w.hidden, j))
        uy, _ = oracle.mxfp4_gemv(*u, w.inter, w.hidden, _one_hot(w.hidden, j))
        assert np.array_equal(out["g"], gy) and np.array_equal(out["u"], uy)
        want = np.array([oracle.silu(a) * b for a, b in zip(gy[0], uy[0])])
        assert np.array_equal(out["h"][0], want)
        swapped = np.array([oracle.silu(b) * a for a, b in zip(gy[0], uy[0])])
        assert not np.allclose(out["h"][0], swapped)


def test_gateup_up_scale_doubling_doubles_h():
    w = workloads.TINY
    g, u = workloads.gateup(w)
    x = workloads.activations(w.wid, 0, 1, w.hidden)
    a = oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, x)
    u2 = (u[0], u[1] + 1, u[2])
    b = oracle.mxfp4_gateup_swiglu(g, u2, w.inter, w.hidden, x)
    assert np.array_equal(b["h"], 2 * a["h"])
    assert np.array_equal(b["g"], a["g"])


def test_gateup_openmp_timing_build_gives_the_same_bits():
    """The benchmark times an OpenMP build of the same row loops: every
    output, magnitude and partial must match the plain build bit for bit."""
    w = workloads.Workload(9, "omp", 512, 300)
    g, u = workloads.gateup(w, 0)
    x = workloads.activations(w.wid, 0, 2, w.hidden)
    a = oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, x)
    b = oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, x, parallel=True)
    assert oracle.threads() == 1
    for k in a:
        assert np.array_equal(a[k].view(np.uint64), b[k].view(np.uint64)), k


def test_route_topk_matches_stable_sort_and_softmax():
    gen = np.random.default_rng(0)
    for trial in range(50):
        n_exp = int(gen.choice([8, 32, 64]))
        topk = int(gen.integers(1, min(8, n_exp) + 1))
        vals = gen.standard_normal((3, n_exp)).astype(np.float32)
        if trial % 2:
            # plant ties: quantise hard so many logits coincide
            vals = np.round(vals * 2) / 2
        lg = workloads.bf16_bits(vals)
        ids, w = oracle.moe_route_topk(lg, topk)
        f = workloads.bf16_to_f32(lg).astype(np.float64)
        for b in range(3):
            order = np.argsort(-f[b], kind="stable")[:topk]
            assert np.array_equal(ids[b], order)
            ref = softmax(f[b][order])
            assert np.allclose(w[b], ref, rtol=1e-14, atol=0)
            # equals the full softmax renormalised over the selection
            full = softmax(f[b])[order]
            assert np.allclose(w[b], full / full.sum(), rtol=1e-13, atol=0)


def test_route_ties_go_to_lower_index():
    lg = workloads.bf16_bits(np.array([[0.5, 1.0, 1.0, 0.25, 1.0, -2.0]], np.float32))
    ids, w = oracle.moe_route_topk(lg, 3)
    assert ids.tolist() == [[1, 2, 4]]
    assert np.allclose(w, 1.0 / 3.0, rtol=1e-15)


def _tiny_moe(n_exp=5, inter=64, hidden=96, seed=0):
    w = workloads.Workload(9, "t", hidden, inter, n_experts=n_exp, topk=2)
    gb = workloads.expert_bank(w, 0, "gate", seed=seed)
    ub = workloads.expert_bank(w, 0, "up", seed=seed)
    db = workloads.expert_bank(w, 0, "down", seed=seed)
    return w, gb, ub, db


def test_moe_gateup_equals_dense_on_each_selected_expert():
    w, gb, ub, _ = _tiny_moe()
    x = workloads.activations(w.wid, 0, 2, w.hidden)
    ids = np.array([[3, 0], [4, 3]], np.int32)
    h, Sg, Su = oracle.moe_gateup_swiglu(gb, ub, w.n_experts, w.inter, w.hidden, x, ids)
    for b in range(2):
        for j in range(2):
            e = ids[b, j]
            d = oracle.mxfp4_gateup_swiglu((gb[0][e], gb[1][e], gb[2][e]),
                                           (ub[0][e], ub[1][e], ub[2][e]),
                                           w.inter, w.hidden, x[b])
            assert np.array_equal(h[b, j], d["h"][0])
            assert np.array_equal(Sg[b, j], d["Sg"][0])


def test_moe_gateup_bad_id_gives_nan_row():
    w, gb, ub, _ = _tiny_moe()
    x = workloads.activations(w.wid, 0, 1, w.hidden)
    ids = np.array([[1, 5]], np.int32)
    h, _, _ = oracle.moe_gateup_swiglu(gb, ub, w.n_experts, w.inter, w.hidden, x, ids)
    assert np.all(np.isfinite(h[0, 0])) and np.all(np.isnan(h[0, 1]))


def test_moe_down_combine_exact_rational():
    """Tiny bank, exact rational evaluation of sum_j w_j * ps * (Wd h_j)."""
    w, _, _, db = _tiny_moe(n_exp=3, inter=32, hidden=32)
    gen = np.random.default_rng(2)
    h = gen.standard_normal((1, 2, 32)).astype(np.float32)
    ids = np.array([[2, 0]], np.int32)
    wt = np.array([[0.625, 0.375]])
    y, S = oracle.moe_down_combine(db, 3, 32, 32, h, ids, wt)
    deq = [oracle.mxfp4_dequantize(db[0][e], db[1][e], 32, 32) for e in range(3)]
    for r in range(32):
        acc = Fraction(0)
        for j in range(2):
            e = ids[0, j]
            dot = sum(Fraction(float(deq[e][r, k])) * Fraction(float(h[0, j, k]))
                      for k in range(32))
            acc += Fraction(wt[0, j]) * Fraction(float(db[2][e][r])) * dot
        assert abs(Fraction(y[0, r]) - acc) <= Fraction(70 * 2.0 ** -53 * S[0, r])


def test_moe_down_combine_special_cases():
    w, _, _, db = _tiny_moe()
    gen = np.random.default_rng(4)
    h = gen.standard_normal((1, 2, w.inter)).astype(np.float32)
    # k = 1, weight 1 -> the plain postscaled matvec of that expert
    y1, _ = oracle.moe_down_combine(db, w.n_experts, w.hidden, w.inter,
                                    h[:, :1], np.array([[2]], np.int32), np.ones((1, 1)))
    e = 2
    deq = oracle.mxfp4_dequantize(db[0][e], db[1][e], w.hidden, w.inter).astype(np.float64)
    ref = db[2][e].astype(np.float64) * (deq @ h[0, 0].astype(np.float64))
    assert np.allclose(y1[0], ref, rtol=1e-12, atol=1e-12)
    # permuting the bank together with the ids leaves y unchanged
    ids = np.array([[4, 1]], np.int32)
    wt = np.array([[0.7, 0.3]])
    ya, _ = oracle.moe_down_combine(db, w.n_experts, w.hidden, w.inter, h, ids, wt)
    perm = np.array([3, 4, 0, 2, 1])   # new slot i holds old expert perm[i]
    inv = np.argsort(perm)
    dbp = tuple(a[perm] for a in db)
    yb, _ = oracle.moe_down_combine(dbp, w.n_experts, w.hidden, w.inter, h,
                                    inv[ids].astype(np.int32), wt)
    assert np.array_equal(ya, yb)
    # a bad id poisons the row
    yc, _ = oracle.moe_down_combine(db, w.n_experts, w.hidden, w.inter, h,
                                    np.array([[4, 9]], np.int32), wt)
    assert np.all(np.isnan(yc))
