"""FP8 E4M3 row-scaled matvec on the device vs the CPU oracle, through the
C ABI: bit-exact decode, then the matvec element by element within the
propagated tolerance, on small ragged shapes and on the SmolLM3- and
Phi-4-shaped down projections (every row), with fp32 and bf16
activations, several batch sizes and bf16 output; and chained after the
MXFP4 gate/up SwiGLU as the dense down projection."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import assert_parity, dev_bf16, dev_u8, gemv_tol, guarded, to_np

pytestmark = pytest.mark.gpu


def test_fp8_dequantize_all_codes_bit_exact(dev):
    n, k = 24, 256
    codes = ((np.arange(k)[None, :] + 37 * np.arange(n)[:, None]) % 256).astype(np.uint8)
    scale = np.linspace(0.25, 4.0, n).astype(np.float32)
    packed = dev_u8(tt.pack_fp8_matrix(codes, scale, n, k), dev)
    w, sc = tt.fp8_dequantize(packed, n, k)
    torch.cuda.synchronize()
    got = w.cpu().numpy()
    ref = np.vectorize(oracle.fp8e4m3_value)(codes.astype(np.int64)).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(to_np(sc), scale)


def _case(dev, n, k, batch, xf32, rows=None, out_dtype=torch.float32, seed=0):
    codes, scale = workloads.fp8_matrix(7, seed, n, k)
    if xf32:
        xh = workloads.swiglu_like(7, seed, batch, k)
        xd = torch.from_numpy(xh).to(dev)
    else:
        xh = workloads.activations(7, seed, batch, k)
        xd = dev_bf16(xh, dev)
    packed = dev_u8(tt.pack_fp8_matrix(codes, scale, n, k), dev)
    y, check = guarded((batch, n), out_dtype, dev)
    tt.fp8_gemv(packed, n, k, xd, out=y)
    check()
    got = to_np(y)
    ref, S = oracle.fp8_gemv(codes, scale, n, k, xh, rows=rows)
    if rows is not None:
        got = got[:, rows]
    return got, ref, S


@pytest.mark.parametrize("n,k,batch,xf32", [(13, 200, 1, True), (8, 128, 1, False),
                                            (100, 1000, 3, False), (40, 4096, 8, True),
                                            (17, 2880, 32, False), (333, 11008, 2, True),
                                            (9, 32768, 1, True), (9, 32768, 1, False),
                                            (5, 16384, 4, False), (1, 8, 1, False)])
def test_fp8_gemv_ragged(dev, n, k, batch, xf32):
    got, ref, S = _case(dev, n, k, batch, xf32)
    assert_parity(got, ref, gemv_tol(S, ref), f"fp8 n{n} k{k} b{batch} {'f32' if xf32 else 'bf16'}")


@pytest.mark.parametrize("xf32", [True, False])
def test_fp8_smollm3_down(dev, xf32):
    n, k = 2048, 11008
    got, ref, S = _case(dev, n, k, 1, xf32)
    assert_parity(got, ref, gemv_tol(S, ref), f"fp8 smollm3 down {'f32' if xf32 else 'bf16'}")


def test_fp8_phi4_down_and_bf16_out(dev):
    n, k = 5120, 17920
    got, ref, S = _case(dev, n, k, 1, False, out_dtype=torch.bfloat16)
    assert_parity(got, ref, gemv_tol(S, ref, bf16=True), "fp8 phi4 down bf16 out (all rows)")


def test_fp8_down_after_gateup(dev):
    """MXFP4 gate/up SwiGLU -> h (fp32) -> FP8 down: the down stage matches
    the oracle on the device's own h."""
    w = workloads.Workload(1, "chain", 2048, 1024)
    g, u = workloads.gateup(w, 0)
    x = workloads.activations(w.wid, 0, 2, w.hidden)
    pg = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    h = tt.mxfp4_gateup_swiglu(pg, w.inter, w.hidden, dev_bf16(x, dev))
    codes, scale = workloads.fp8_matrix(7, 3, w.hidden, w.inter)
    pd = dev_u8(tt.pack_fp8_matrix(codes, scale, w.hidden, w.inter), dev)
    y = tt.fp8_gemv(pd, w.hidden, w.inter, h)
    torch.cuda.synchronize()
    ref, S = oracle.fp8_gemv(codes, scale, w.hidden, w.inter, to_np(h))
    assert_parity(to_np(y), ref, gemv_tol(S, ref), "fp8 down after gate/up")


def test_fp8_run_to_run_bit_identical(dev):
    n, k = 512, 4096
    codes, scale = workloads.fp8_matrix(7, 4, n, k)
    packed = dev_u8(tt.pack_fp8_matrix(codes, scale, n, k), dev)
    x = torch.from_numpy(workloads.swiglu_like(7, 4, 4, k)).to(dev)
    a = tt.fp8_gemv(packed, n, k, x)
    b = tt.fp8_gemv(packed, n, k, x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
