"""The allocation-free attention entry point (tt_gqa_attention_decode_noalloc,
through the C ABI) against the workspace entry point it mirrors: the same
bits on two calls in a row, the second with a smaller context, both also
within the oracle's bound; a call that needs more partials than the
library's per-device array is refused with TT_E_SIZE; and the call leaves
the device's free memory unchanged."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import assert_parity, dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _inputs(dev, hq, hkv, d, tcap, seed):
    gen = np.random.default_rng(seed)
    q = workloads.bf16_bits(gen.standard_normal((hq, d)).astype(np.float32))
    K = workloads.bf16_bits(gen.standard_normal((hkv, tcap, d)).astype(np.float32))
    V = workloads.bf16_bits(gen.standard_normal((hkv, tcap, d)).astype(np.float32))
    return (q, K, V), (dev_bf16(q, dev), dev_bf16(K, dev), dev_bf16(V, dev))


@pytest.mark.parametrize("hq,hkv,d,T1,T2", [(40, 10, 128, 4096, 700), (64, 8, 64, 2049, 100)])
def test_noalloc_attention_matches_workspace_call(dev, hq, hkv, d, T1, T2):
    (qh, Kh, Vh), (q, K, V) = _inputs(dev, hq, hkv, d, T1, hq + T1)
    scale = d ** -0.5
    out = torch.empty((hq, d), dtype=torch.float32, device=dev)
    for T in (T1, T2):      # the second call is smaller: fewer, or shorter, chunks
        want = tt.gqa_attention_decode(q, K, V, hq, hkv, d, T, scale)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        tt.gqa_attention_decode_noalloc(q, K, V, hq, hkv, d, T, scale, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0, "the call changed the free device memory"
        assert torch.equal(out, want), f"T = {T}: differs from the workspace entry point"
        ref, A, Smax = oracle.gqa_attention(qh, Kh, Vh, hq, hkv, d, T1, T, scale)
        tol = (2e-3 + 4e-5 * Smax[:, None]) * A
        assert_parity(to_np(out), ref, tol, f"no-alloc attention hq{hq} d{d} T{T}")


def test_noalloc_attention_refuses_oversized_calls(dev):
    hq, hkv, d = 40, 10, 128
    T = 1 << 16      # 1024 chunks x 40 heads x 130 floats > 8 MiB
    assert tt.gqa_attention_workspace_bytes(hq, hkv, d, T) > 8 << 20
    (_, _, _), (q, K, V) = _inputs(dev, hq, hkv, d, 64, 3)
    with pytest.raises(tt.TTError) as e:
        tt.gqa_attention_decode_noalloc(q, K, V, hq, hkv, d, T, 0.1)
    assert e.value.status == -5   # TT_E_SIZE, nothing launched
