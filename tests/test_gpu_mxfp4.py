"""GPU parity of the MXFP4 gate/up SwiGLU path (dense, batch 1..32) and of the
MXFP4 decode, against the CPU oracle, through the C ABI.  The full-size
configs are checked on every output row (the large ones against the OpenMP
build of the oracle, pinned bit for bit to the plain build by a CPU test)."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import (REL, assert_parity, dev_bf16, dev_u8, guarded, h_tol, to_np)

pytestmark = pytest.mark.gpu


def _f32_bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _gateup_case(dev, w, layer, batch, rows=None, out_dtype=torch.float32, g=None, u=None,
                 x=None, guard=False):
    if g is None:
        g, u = workloads.gateup(w, layer)
    if x is None:
        x = workloads.activations(w.wid, layer, batch, w.hidden)
    packed = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    out, check = (guarded((batch, w.inter), out_dtype, dev) if guard else (None, None))
    h = tt.mxfp4_gateup_swiglu(packed, w.inter, w.hidden, dev_bf16(x, dev), out=out,
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    if check:
        check()
    got = to_np(h)
    # large cases use the OpenMP build of the oracle (same loops, same bits)
    big = batch * w.inter * w.hidden > 64 << 20
    ref = oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, x, rows=rows, parallel=big)
    if rows is not None:
        got = got[:, rows]
    return got, ref


# ---- decode, bit-exact --------------------------------------------------------

@pytest.mark.parametrize("n,k", [(40, 256), (33, 2880), (16, 96), (7, 32)])
def test_mxfp4_dequantize_bit_exact_all_scale_bytes(dev, n, k):
    gen = np.random.default_rng([n, k])
    codes = gen.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = gen.integers(0, 256, (n, k // 32), dtype=np.uint8)
    flat = scales.reshape(-1)
    flat[: min(256, flat.size)] = np.arange(min(256, flat.size), dtype=np.uint8)
    ps = gen.uniform(0.5, 1.5, n).astype(np.float32)
    packed = dev_u8(tt.pack_mxfp4_matrix(codes, scales, ps, n, k), dev)
    w, p = tt.mxfp4_dequantize(packed, n, k)
    torch.cuda.synchronize()
    got = w.cpu().numpy()
    ref = oracle.mxfp4_dequantize(codes, scales, n, k)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(_f32_bits(got)[~nan], _f32_bits(ref)[~nan])
    assert np.array_equal(p.cpu().numpy(), ps)


def test_mxfp4_every_code_times_every_scale(dev):
    """Row e holds every code twice under scale byte e: 256 x 16 pairs."""
    n, k = 256, 32
    codes = np.tile(np.array([c | (c << 4) for c in range(16)], np.uint8), (n, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(n, 1)
    packed = dev_u8(tt.pack_mxfp4_matrix(codes, scales, None, n, k), dev)
    w, _ = tt.mxfp4_dequantize(packed, n, k)
    got = w.cpu().numpy()
    for e in range(256):
        for c in range(16):
            want = oracle.mxfp4_weight(c, e)
            for j in (2 * c, 2 * c + 1):
                if np.isnan(want):
                    assert np.isnan(got[e, j])
                else:
                    assert _f32_bits(got[e, j]) == _f32_bits(want), (e, c)


def test_gateup_dequantize_bit_exact(dev):
    w = workloads.Workload(9, "t", 2880, 100)
    g, u = workloads.gateup(w)
    packed = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    gd, ud, gp, up = tt.mxfp4_gateup_dequantize(packed, w.inter, w.hidden)
    for (c, s, p), d, dp in ((g, gd, gp), (u, ud, up)):
        ref = oracle.mxfp4_dequantize(c, s, w.inter, w.hidden)
        assert np.array_equal(_f32_bits(d.cpu().numpy()), _f32_bits(ref))
        assert np.array_equal(dp.cpu().numpy(), p)


# ---- gate/up SwiGLU -------------------------------------------------------------

def test_tiny_config_full(dev):
    w = workloads.TINY
    got, ref = _gateup_case(dev, w, 0, 1)
    assert_parity(got, ref["h"], h_tol(ref), "tiny h256 i512 b1")


@pytest.mark.parametrize("hidden,inter", [(32, 8), (96, 100), (2880, 37), (160, 1), (5120, 24),
                                          (2880, 1024), (3200, 520), (2336, 1000), (16384, 40)])
def test_ragged_shapes(dev, hidden, inter):
    w = workloads.Workload(9, "ragged", hidden, inter)
    got, ref = _gateup_case(dev, w, 0, 1, guard=True)
    assert_parity(got, ref["h"], h_tol(ref), f"ragged h{hidden} i{inter}")


def test_smollm3_all_layers_every_row(dev):
    """The SmolLM3-3B-shaped config: all 24 layers, every output row."""
    w = workloads.SMOLLM3
    for layer in range(w.layers):
        got, ref = _gateup_case(dev, w, layer, 1)
        assert_parity(got, ref["h"], h_tol(ref), f"smollm3 layer {layer} (all {w.inter} rows)")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_many_tiles_every_row(dev, out_dtype):
    """More tiles than the chip holds at once at K = 5120 (1125 ten-wave
    tiles), every row checked."""
    w = workloads.Workload(9, "wide", 5120, 9000)
    got, ref = _gateup_case(dev, w, 0, 1, out_dtype=out_dtype)
    assert_parity(got, ref["h"], h_tol(ref, bf16=out_dtype == torch.bfloat16),
                  f"h5120 i9000 {out_dtype}")


def test_phi4_gateup_every_row(dev):
    """The Phi-4-shaped gate/up (hidden 5120, inter 17920), every row."""
    w = workloads.PHI4
    got, ref = _gateup_case(dev, w, 0, 1)
    assert_parity(got, ref["h"], h_tol(ref), f"phi4 gate/up (all {w.inter} rows)")


@pytest.mark.parametrize("batch", [2, 4, 8, 16, 17, 32])
def test_batched_smollm3_every_row(dev, batch):
    """The batched config (SmolLM3 shapes) at each batch, every row."""
    w = workloads.BATCHED
    got, ref = _gateup_case(dev, w, 0, batch)
    assert_parity(got, ref["h"], h_tol(ref), f"batched b{batch} (all rows)")


# MFMA path off the SmolLM3 shape: ragged last unit (qv_last < 4), two chunks
# per tile, a single unit, tiles past the grid (each wave walks several
# tiles), widths that fall back to one weight pass per token, workgroups
# that own more tiles than a row has K-chunks (the finishing waves of the
# later tiles never enter the K loop), 32-token-path runs shorter than
# the longest allowed (2 and 5 tiles per workgroup, the second with 9
# K-chunks, so two rounds of tile fetches), and six-tile runs of one
# 16-token block (2048 tiles: more workgroups than CUs; 9 K-chunks).
@pytest.mark.parametrize("hidden,inter,batch", [(2880, 1000, 5), (4096, 520, 9), (2336, 1000, 32),
                                                (96, 100, 3), (32, 8, 2), (5120, 24, 4),
                                                (2048, 20000, 32), (2048, 11008, 23),
                                                (256, 8192, 4), (1024, 16384, 20),
                                                (256, 16384, 32), (512, 12000, 9),
                                                (2880, 1001, 17), (96, 37, 5), (160, 1, 3),
                                                (1024, 1002, 32), (512, 3000, 24),
                                                (2304, 8200, 20), (1024, 16384, 12),
                                                (2304, 3000, 16)])
def test_batched_ragged_shapes(dev, hidden, inter, batch):
    w = workloads.Workload(9, "ragged", hidden, inter)
    got, ref = _gateup_case(dev, w, 0, batch, guard=True)
    assert_parity(got, ref["h"], h_tol(ref), f"batched ragged h{hidden} i{inter} b{batch}")


@pytest.mark.parametrize("batch,inter", [(1, 300), (8, 300), (8, 301), (32, 302)])
def test_bf16_output(dev, batch, inter):
    # odd and 2-mod-4 row lengths put rows off the 8-byte alignment of the
    # batched kernel's 4-output stores (the element-wise fallback)
    w = workloads.Workload(9, "bf16", 512, inter)
    got, ref = _gateup_case(dev, w, 0, batch, out_dtype=torch.bfloat16, guard=True)
    assert_parity(got, ref["h"], h_tol(ref, bf16=True), f"bf16 out b{batch}")


@pytest.mark.parametrize("batch,out_dtype", [(8, torch.float32), (32, torch.float32),
                                             (8, torch.bfloat16)])
def test_batched_output_off_alignment(dev, batch, out_dtype):
    """An output that starts one element past an aligned address: the
    batched kernel's 4-output stores must fall back to element stores."""
    w = workloads.Workload(9, "offal", 1024, 400)
    g, u = workloads.gateup(w)
    x = workloads.activations(w.wid, 0, batch, w.hidden)
    packed = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    buf = torch.full((batch * w.inter + 2,), 7.0, dtype=out_dtype, device=dev)
    out = buf[1:1 + batch * w.inter].view(batch, w.inter)
    tt.mxfp4_gateup_swiglu(packed, w.inter, w.hidden, dev_bf16(x, dev), out=out,
                           out_dtype=out_dtype)
    torch.cuda.synchronize()
    ends = buf[[0, -1]].float().cpu().numpy()
    assert np.all(ends == 7.0), "element before or after the output was overwritten"
    ref = oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, x)
    assert_parity(to_np(out), ref["h"], h_tol(ref, bf16=out_dtype == torch.bfloat16),
                  f"offset output b{batch}")


@pytest.mark.parametrize("batch", [1, 2, 16, 32])
def test_up_scale_doubling_is_exact(dev, batch):
    """Up scale bytes e -> e+1 doubles u exactly and leaves silu(g)
    unchanged, so h doubles bit for bit (on the device alone)."""
    w = workloads.Workload(9, "dbl", 1024, 200)
    g, u = workloads.gateup(w)
    x = workloads.activations(w.wid, 0, batch, w.hidden)
    xd = dev_bf16(x, dev)
    p1 = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    p2 = dev_u8(tt.pack_mxfp4_gateup(g, (u[0], u[1] + 1, u[2]), w.inter, w.hidden), dev)
    h1 = tt.mxfp4_gateup_swiglu(p1, w.inter, w.hidden, xd)
    h2 = tt.mxfp4_gateup_swiglu(p2, w.inter, w.hidden, xd)
    assert torch.equal(h2, 2 * h1)


@pytest.mark.parametrize("batch", [1, 8])
def test_run_to_run_bit_identical(dev, batch):
    w = workloads.SMOLLM3
    g, u = workloads.gateup(w, 3)
    x = dev_bf16(workloads.activations(w.wid, 3, batch, w.hidden), dev)
    packed = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    a = tt.mxfp4_gateup_swiglu(packed, w.inter, w.hidden, x)
    b = tt.mxfp4_gateup_swiglu(packed, w.inter, w.hidden, x)
    assert torch.equal(a, b)


def test_one_hot_up_column_gives_silu_of_gate(dev):
    """Up column j is code 2 (1.0) under scale 127 with postscale 1 and every
    other up code 0; x = e_j makes u = 1 exactly, so h = silu(ps_g w_g[:, j])."""
    w = workloads.Workload(9, "onehot", 256, 64)
    g, _ = workloads.gateup(w)
    j = 77
    uc = np.zeros((w.inter, w.hidden // 2), np.uint8)
    uc[:, j // 2] = 2 << 4 if j & 1 else 2
    us = np.full((w.inter, w.hidden // 32), 127, np.uint8)
    u = (uc, us, np.ones(w.inter, np.float32))
    x = np.zeros((1, w.hidden), np.uint16)
    x[0, j] = 0x3F80
    got, ref = _gateup_case(dev, w, 0, 1, g=g, u=u, x=x)
    assert np.all(ref["u"] == 1.0)
    assert_parity(got, ref["h"], 4e-7 * np.abs(ref["h"]) + 1e-30, "one-hot up column")


@pytest.mark.parametrize("batch", [1, 4])
def test_quantized_fp32_weights_end_to_end(dev, batch):
    """fp32 gate and up rows through the library's MXFP4 quantizer (with the
    fitted row postscale), packed and run on the device: parity with the
    oracle on the same codes.  The device decode of the packed gate rows,
    scaled by the fitted postscale, is closer to the fp32 rows than the
    decode alone, row by row (what a least-squares postscale guarantees)."""
    gen = np.random.default_rng(31)
    inter, hidden = 1000, 2048
    wg = (0.02 * gen.standard_normal((inter, hidden))).astype(np.float32)
    wu = (0.02 * gen.standard_normal((inter, hidden))).astype(np.float32)
    w = workloads.Workload(9, "quantized", hidden, inter)
    x = workloads.activations(9, 0, batch, hidden)
    g, u = tt.quantize_mxfp4(wg), tt.quantize_mxfp4(wu)
    got, ref = _gateup_case(dev, w, 0, batch, g=g, u=u, x=x)
    assert_parity(got, ref["h"], h_tol(ref), f"quantized b{batch}")
    packed = dev_u8(tt.pack_mxfp4_matrix(g[0], g[1], g[2], inter, hidden), dev)
    d, ps = tt.mxfp4_dequantize(packed, inter, hidden)
    torch.cuda.synchronize()
    d, ps = to_np(d).astype(np.float64), to_np(ps)
    assert np.array_equal(ps, g[2])
    e_fit = ((wg - ps[:, None] * d) ** 2).sum(axis=1)
    e_one = ((wg - d) ** 2).sum(axis=1)
    assert np.all(e_fit <= e_one * (1 + 1e-12))


def _wide_range_bf16(gen, shape, lo=-40, hi=12):
    """bf16 activations with magnitudes 2^U(lo, hi) and random signs: every
    32-element block spans far more than the 2^13 its two E4M3 parts carry
    exactly, so the small elements exercise the lo part's rounding, and zeros
    and exact powers of two are mixed in."""
    mag = np.exp2(gen.uniform(lo, hi, shape))
    sign = np.where(gen.random(shape) < 0.5, -1.0, 1.0)
    x = (sign * mag).astype(np.float32)
    x[gen.random(shape) < 0.05] = 0.0
    pw = gen.random(shape) < 0.05
    x[pw] = np.exp2(np.round(gen.uniform(lo, hi, int(pw.sum())))).astype(np.float32)
    return workloads.bf16_bits(x)


@pytest.mark.parametrize("batch", [1, 2])
def test_wide_range_activations(dev, batch):
    """Activations spread over 2^52 within every block, through the two-part
    E4M3 split of the scaled-MFMA path: parity at the usual bar."""
    w = workloads.Workload(9, "wide", 2048, 640)
    x = _wide_range_bf16(np.random.default_rng(77 + batch), (batch, w.hidden))
    got, ref = _gateup_case(dev, w, 0, batch, x=x)
    assert_parity(got, ref["h"], h_tol(ref), f"wide-range x b{batch}")


def test_block_exponent_extremes(dev):
    """Blocks whose largest element sits at the top and at the bottom of the
    bf16 normal range (the split's scale byte clamps) and an all-zero block:
    parity at the usual bar, no overflow or NaN."""
    w = workloads.Workload(9, "ext", 256, 128)
    x = np.zeros((1, w.hidden), np.float32)
    x[0, 0:32] = np.float32(2.0 ** 120) * np.linspace(-1, 1, 32, dtype=np.float32)
    x[0, 32:64] = np.float32(2.0 ** -120) * np.linspace(1, 2, 32, dtype=np.float32)
    x[0, 96:128] = np.float32(3.0) * np.float32(2.0 ** -126)     # smallest normals
    x[0, 128:160] = np.float32(1.0)
    # gate/up values near 2^120 would overflow silu * up; scale those columns
    # to zero weight so the rows stay finite: the test is about the split
    g, u = workloads.gateup(w)
    for cu in (g, u):
        cu[0][:, 0:16] = 0
    got, ref = _gateup_case(dev, w, 0, 1, g=g, u=u, x=workloads.bf16_bits(x))
    assert np.all(np.isfinite(got))
    assert_parity(got, ref["h"], h_tol(ref), "block exponent extremes")


# ---- E8M0 0xFF (NaN) blocks on every path ----------------------------------------

@pytest.mark.parametrize("batch", [1, 2, 8, 32])
def test_nan_scale_blocks(dev, batch):
    """A block whose E8M0 byte is 0xFF decodes to NaN (OCP MX): every output
    row that reads one (in its gate or its up row) is NaN, every other row
    matches the oracle.  Covers the scaled-MFMA path (batch 1, 2) and the
    bf16-MFMA path (batch 8, 32), with NaN blocks in the first, a middle and
    the last block of a row, and a row whose activations over the NaN block
    are zero (NaN times zero is still NaN)."""
    w = workloads.Workload(9, "nanblk", 1024, 200)
    g, u = workloads.gateup(w)
    gs, us = g[1].copy(), u[1].copy()
    nb = w.hidden // 32
    for r, blk in ((0, 0), (5, nb // 2), (17, nb - 1), (40, 3), (199, 7)):
        gs[r, blk] = 0xFF
    for r, blk in ((9, 1), (17, 2), (120, nb - 1), (150, 0)):
        us[r, blk] = 0xFF
    x = workloads.activations(w.wid, 0, batch, w.hidden)
    x[:, 3 * 32:4 * 32] = 0   # row 40's NaN block meets zero activations
    got, ref = _gateup_case(dev, w, 0, batch, g=(g[0], gs, g[2]), u=(u[0], us, u[2]), x=x,
                            guard=True)
    nan_rows = {0, 5, 17, 40, 199, 9, 120, 150}
    assert set(np.where(np.isnan(ref["h"][0]))[0].tolist()) == nan_rows
    assert_parity(got, ref["h"], h_tol(ref), f"NaN scale blocks b{batch}")


# ---- accumulation of the scaled FP4 x FP8 instruction, worst case --------------------

def _spread_rows(inter, hidden, seed):
    """Gate rows whose products span a wide range inside every 128-element
    block of K (one matrix instruction adds 128 products):

    rows 0..39: in each 128-block, one large product (code 6 under scale
      byte e0) and 96 small ones of the same sign (code 0.5 under e0 - d) in
      the other three 32-element blocks; d = r runs 0..39, so the small
      products sit 2^-3.6 .. 2^-43 below the large one and the sweep crosses
      whatever alignment window the instruction keeps;
    rows 40..47: the same with the small products of the opposite sign;
    rows 48..63: random codes under scale bytes drawn per block from
      e0 - 40 .. e0, and random signs.
    Up rows are 1.0 at one column under scale 127 (u = x there), so h is
    silu(g) times that activation."""
    gen = np.random.default_rng(seed)
    nb = hidden // 32
    e0 = 127
    codes = np.zeros((inter, hidden), np.uint8)
    scales = np.full((inter, nb), e0, np.uint8)
    for r in range(48):
        d = r if r < 40 else 4 + 4 * (r - 40)
        neg = r >= 40
        for b in range(0, nb, 4):
            codes[r, 32 * b] = 7                               # +6 * 2^0
            codes[r, 32 * (b + 1):32 * (b + 4)] = 9 if neg else 1   # -/+0.5
            scales[r, b + 1:b + 4] = e0 - d
    codes[48:] = gen.integers(0, 16, (inter - 48, hidden), dtype=np.uint8)
    scales[48:] = gen.integers(e0 - 40, e0 + 1, (inter - 48, nb), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, np.ones(inter, np.float32)


@pytest.mark.parametrize("batch", [1, 2, 8])
def test_accumulation_worst_case_k16384(dev, batch):
    """K = 16384 with the products of every 128-element block spread over up
    to 2^43 (see _spread_rows), activations either all 1.5 (exact in one
    E4M3 part) or random bf16 spread over 2^-8 .. 2^8: every row within
    2e-3 * sum |w x| of the oracle.  Batch 1 and 2 run on the scaled FP4 x
    FP8 instruction, batch 8 on the bf16 matrix cores (for comparison).  The
    worst err/tol is printed."""
    hidden, inter = 16384, 64
    w = workloads.Workload(9, "spread", hidden, inter)
    g = _spread_rows(inter, hidden, 3)
    uc = np.zeros((inter, hidden // 2), np.uint8)
    uc[:, 0] = 2                                             # column 0: 1.0
    u = (uc, np.full((inter, hidden // 32), 127, np.uint8), np.ones(inter, np.float32))
    gen = np.random.default_rng(4)
    x1 = np.full((batch, hidden), 1.5, np.float32)
    mag = np.exp2(gen.uniform(-8, 8, (batch, hidden)))
    x2 = (np.where(gen.random((batch, hidden)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    worst = 0.0
    for name, xf in (("x=1.5", x1), ("x spread", x2)):
        xf[:, 0] = 1.0                                       # u = 1 exactly
        got, ref = _gateup_case(dev, w, 0, batch, g=g, u=u, x=workloads.bf16_bits(xf))
        tol = h_tol(ref)
        err = np.abs(got - ref["h"])
        worst = max(worst, float((err / tol).max()))
        assert_parity(got, ref["h"], tol, f"worst-case accumulation K=16384 b{batch} {name}")
    print(f"K=16384 b{batch}: worst err/tol {worst:.3e} (REL = {REL})")
