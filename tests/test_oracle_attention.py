"""Pins of the CPU oracle's single-token GQA attention (no GPU).

Pinned against an independent numpy/scipy formulation, closed forms (one
cached position; identical keys; one dominant key), the GQA head mapping
(equal to multi-head attention with repeated kv heads) and exact
invariants (scale moved between the keys and the scale factor; token
order).
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads


def _cache(gen, hq, hkv, d, tcap, T):
    q = workloads.bf16_bits(gen.standard_normal((hq, d)).astype(np.float32))
    K = workloads.bf16_bits(gen.standard_normal((hkv, tcap, d)).astype(np.float32))
    V = workloads.bf16_bits(gen.standard_normal((hkv, tcap, d)).astype(np.float32))
    return q, K, V


def _numpy_attention(q, K, V, hq, hkv, T, scale):
    qf = workloads.bf16_to_f32(q).astype(np.float64)
    Kf = workloads.bf16_to_f32(K).astype(np.float64)[:, :T]
    Vf = workloads.bf16_to_f32(V).astype(np.float64)[:, :T]
    g = np.arange(hq) // (hq // hkv)
    s = np.einsum("htd,hd->ht", Kf[g], qf) * scale
    p = softmax(s, axis=1)
    return np.einsum("ht,htd->hd", p, Vf[g])


@pytest.mark.parametrize("hq,hkv,d,tcap,T", [(8, 2, 64, 40, 33), (40, 10, 128, 300, 257),
                                             (4, 4, 128, 16, 16), (6, 1, 32, 9, 9)])
def test_attention_matches_numpy_scipy(hq, hkv, d, tcap, T):
    gen = np.random.default_rng(hq * 1000 + T)
    q, K, V = _cache(gen, hq, hkv, d, tcap, T)
    scale = 1.0 / np.sqrt(d)
    out, A, _ = oracle.gqa_attention(q, K, V, hq, hkv, d, tcap, T, scale)
    ref = _numpy_attention(q, K, V, hq, hkv, T, scale)
    assert np.all(np.abs(out - ref) <= 1e-12 * (A + 1e-300))


def test_one_position_returns_its_value_exactly():
    gen = np.random.default_rng(1)
    q, K, V = _cache(gen, 8, 2, 64, 5, 1)
    out, _, _ = oracle.gqa_attention(q, K, V, 8, 2, 64, 5, 1, 0.125)
    want = workloads.bf16_to_f32(V[np.arange(8) // 4, 0]).astype(np.float64)
    assert np.array_equal(out, want)


def test_identical_keys_average_the_values_exactly():
    gen = np.random.default_rng(2)
    hq, hkv, d, T = 4, 2, 32, 16
    q, K, V = _cache(gen, hq, hkv, d, T, T)
    K[:] = K[:, :1]                                     # every key the same
    V = workloads.bf16_bits(gen.integers(-8, 9, (hkv, T, d)).astype(np.float32))
    out, _, _ = oracle.gqa_attention(q, K, V, hq, hkv, d, T, T, 0.2)
    Vf = workloads.bf16_to_f32(V).astype(np.float64)
    assert np.array_equal(out, Vf.mean(axis=1)[np.arange(hq) // 2])


def test_dominant_key_selects_its_value():
    gen = np.random.default_rng(3)
    hq, hkv, d, T = 2, 1, 64, 20
    q, K, V = _cache(gen, hq, hkv, d, T, T)
    q[:] = workloads.bf16_bits(np.ones((hq, d), np.float32))
    K[:] = workloads.bf16_bits(np.zeros((hkv, T, d), np.float32))
    K[0, 7] = workloads.bf16_bits(np.ones(d, np.float32))   # score 64 * 1.0
    out, _, _ = oracle.gqa_attention(q, K, V, hq, hkv, d, T, T, 1.0)
    v7 = workloads.bf16_to_f32(V[0, 7]).astype(np.float64)
    assert np.all(np.abs(out - v7) <= 1e-20 + 1e-15 * np.abs(v7))


def test_gqa_equals_mha_with_repeated_kv_heads():
    gen = np.random.default_rng(4)
    hq, hkv, d, T = 8, 2, 64, 31
    q, K, V = _cache(gen, hq, hkv, d, T, T)
    out, _, _ = oracle.gqa_attention(q, K, V, hq, hkv, d, T, T, 0.125)
    rep = np.arange(hq) // (hq // hkv)
    out2, _, _ = oracle.gqa_attention(q, K[rep], V[rep], hq, hq, d, T, T, 0.125)
    assert np.array_equal(out, out2)


def test_scale_and_token_order_invariants():
    gen = np.random.default_rng(5)
    hq, hkv, d, T = 4, 2, 64, 24
    q, K, V = _cache(gen, hq, hkv, d, T, T)
    out, A, _ = oracle.gqa_attention(q, K, V, hq, hkv, d, T, T, 0.25)
    # halving every key (exact in bf16 away from the subnormal range) and
    # doubling the scale leaves every score, hence the output, unchanged
    Kh = workloads.bf16_bits(workloads.bf16_to_f32(K) * 0.5)
    out2, _, _ = oracle.gqa_attention(q, Kh, V, hq, hkv, d, T, T, 0.5)
    assert np.array_equal(out, out2)
    perm = gen.permutation(T)
    out3, _, _ = oracle.gqa_attention(q, K[:, perm], V[:, perm], hq, hkv, d, T, T, 0.25)
    assert np.all(np.abs(out3 - out) <= 1e-13 * A)
