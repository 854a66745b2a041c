"""Single-token GQA attention on the device vs the CPU oracle, through the C
ABI: Phi-4-shaped heads (40 / 10 x 128) and gpt-oss-shaped heads (64 / 8 x
64) at short and long contexts, ragged T, bf16 output, a cache with spare
capacity, T = 1, and run-to-run identity.

Tolerance: with score errors below 1e-5 * Smax (fp32 sums of 128 products
are good to a few 1e-6 relative) the softmax weights move by at most a
factor exp(±2e-5 Smax), so |out - ref| <= (2e-3 + 4e-5 * Smax) * A,
A = sum_t p_t |V| per element, plus the spec cosine bound."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import assert_parity, dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _case(dev, hq, hkv, d, tcap, T, seed, out_dtype=torch.float32):
    gen = np.random.default_rng(seed)
    q = workloads.bf16_bits(gen.standard_normal((hq, d)).astype(np.float32))
    K = workloads.bf16_bits(gen.standard_normal((hkv, tcap, d)).astype(np.float32))
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
                                        (64, 8, 64, 2049), (8, 8, 128, 300), (4, 2, 64, 65)])
def test_gqa_attention(dev, hq, hkv, d, T):
    got, ref, tol = _case(dev, hq, hkv, d, T, T, hq * 7 + T)
    assert_parity(got, ref, tol, f"attention hq{hq} hkv{hkv} d{d} T{T}")


def test_gqa_attention_spare_capacity_and_bf16_out(dev):
    got, ref, tol = _case(dev, 40, 10, 128, 1000, 777, 5, out_dtype=torch.bfloat16)
    assert_parity(got, ref, tol, "attention tcap 1000 T 777 bf16 out")


def test_gqa_attention_run_to_run_identical(dev):
    gen = np.random.default_rng(9)
    hq, hkv, d, T = 40, 10, 128, 1500
    q = dev_bf16(workloads.bf16_bits(gen.standard_normal((hq, d)).astype(np.float32)), dev)
    K = dev_bf16(workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32)), dev)
    V = dev_bf16(workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32)), dev)
    a = tt.gqa_attention_decode(q, K, V, hq, hkv, d, T, 0.088)
    b = tt.gqa_attention_decode(q, K, V, hq, hkv, d, T, 0.088)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
