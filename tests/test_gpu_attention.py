"""Single-token GQA attention on the device vs the CPU oracle, through the C
ABI: Phi-4-shaped heads (40 / 10 x 128) and gpt-oss-shaped heads (64 / 8 x
64) at short and long contexts, every supported group size G = hq / hkv (1,
2, 4, 8) at d = 64 and 128, ragged T, bf16 output, a cache with spare
capacity, T = 1, scores spread over a wide range, and run-to-run identity.

Tolerance: scores are bf16 x bf16 products (exact in fp32) accumulated in
fp32 on the matrix cores, and the softmax weights enter P V as two bf16
parts (residue 2^-18 relative).  With score errors below 1e-5 * Smax the
weights move by at most a factor exp(+-2e-5 Smax), so |out - ref| <= (2e-3 +
4e-5 * Smax) * A, A = sum_t p_t |V| per element, plus the cosine bound."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import assert_parity, dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _case(dev, hq, hkv, d, tcap, T, seed, out_dtype=torch.float32, q_mul=1.0, k_spread=0):
    gen = np.random.default_rng(seed)
    q = workloads.bf16_bits((q_mul * gen.standard_normal((hq, d))).astype(np.float32))
    kf = gen.standard_normal((hkv, tcap, d))
    if k_spread:
        kf = kf * np.exp2(gen.integers(-k_spread, k_spread + 1, kf.shape))
    K = workloads.bf16_bits(kf.astype(np.float32))
    V = workloads.bf16_bits(gen.standard_normal((hkv, tcap, d)).astype(np.float32))
    scale = 1.0 / np.sqrt(d)
    out = tt.gqa_attention_decode(dev_bf16(q, dev), dev_bf16(K, dev), dev_bf16(V, dev), hq, hkv,
                                  d, T, scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, A, Smax = oracle.gqa_attention(q, K, V, hq, hkv, d, tcap, T, scale)
    tol = (2e-3 + 4e-5 * Smax[:, None]) * A
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    return to_np(out), ref, tol


@pytest.mark.parametrize("hq,hkv,d,T", [(40, 10, 128, 1), (40, 10, 128, 63), (40, 10, 128, 256),
                                        (40, 10, 128, 4096), (64, 8, 64, 100),
                                        (64, 8, 64, 2049), (8, 8, 128, 300), (4, 2, 64, 65),
                                        (32, 4, 128, 517), (16, 16, 64, 33), (16, 8, 128, 1),
                                        (32, 8, 64, 4097), (8, 4, 64, 16), (16, 2, 128, 8192),
                                        (40, 10, 128, 128), (8, 2, 128, 100), (64, 8, 64, 256),
                                        (16, 8, 64, 193)])
def test_gqa_attention(dev, hq, hkv, d, T):
    got, ref, tol = _case(dev, hq, hkv, d, T, T, hq * 7 + T)
    assert_parity(got, ref, tol, f"attention hq{hq} hkv{hkv} d{d} T{T}")


@pytest.mark.parametrize("hq,hkv,d", [(40, 10, 128), (64, 8, 64)])
def test_gqa_attention_wide_range_scores(dev, hq, hkv, d):
    # q x 6 and key elements scaled by 2^-6 .. 2^6: scores of magnitude ~50
    # and products spread over 24 binades inside every dot product
    got, ref, tol = _case(dev, hq, hkv, d, 700, 700, 31 + d, q_mul=6.0, k_spread=6)
    assert_parity(got, ref, tol, f"attention wide-range scores hq{hq} d{d}")


def test_gqa_attention_spare_capacity_and_bf16_out(dev):
    got, ref, tol = _case(dev, 40, 10, 128, 1000, 777, 5, out_dtype=torch.bfloat16)
    assert_parity(got, ref, tol, "attention tcap 1000 T 777 bf16 out")


def test_gqa_attention_single_workgroup_bf16_out(dev):
    # a context that fits one workgroup per kv head, in a larger cache
    got, ref, tol = _case(dev, 64, 8, 64, 600, 230, 11, out_dtype=torch.bfloat16)
    assert_parity(got, ref, tol, "attention tcap 600 T 230 bf16 out (one workgroup)")


def test_gqa_attention_run_to_run_identical(dev):
    gen = np.random.default_rng(9)
    hq, hkv, d, T = 40, 10, 128, 1500
    q = dev_bf16(workloads.bf16_bits(gen.standard_normal((hq, d)).astype(np.float32)), dev)
    K = dev_bf16(workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32)), dev)
    V = dev_bf16(workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32)), dev)
    for t in (T, 100):   # split over chunks, and one workgroup per kv head
        a = tt.gqa_attention_decode(q, K, V, hq, hkv, d, t, 0.088)
        b = tt.gqa_attention_decode(q, K, V, hq, hkv, d, t, 0.088)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
