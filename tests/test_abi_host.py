"""Host-side tests of libtt.so (no GPU): exported symbols, status codes,
packers and the INT4 quantizer."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "tt.h")).read()
    return sorted(set(re.findall(r"\b(tt_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 19
    lib = ctypes.CDLL(tt.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(tt.EXPORTS)


def test_format_info_is_honest():
    assert tt.format_info(tt.TT_FMT_MXFP4) == dict(bits=4, group=32, scale_kind=0, has_zero=0)
    assert tt.format_info(tt.TT_FMT_INT4_AFFINE) == dict(bits=4, group=128, scale_kind=1,
                                                         has_zero=1)
    with pytest.raises(tt.TTError) as e:
        tt.format_info(7)
    assert e.value.status == -4


# Fake but aligned non-null device pointers: validation must reject the call
# before anything touches the device.
P = ctypes.c_void_p(0x10000)


@pytest.mark.parametrize("args,status", [
    ((None, 16, 64, P, 1, P, 0, None), -1),      # null weights
    ((P, 16, 48, P, 1, P, 0, None), -2),         # hidden not a multiple of 32
    ((P, 16, 64, P, 0, P, 0, None), -2),         # batch 0
    ((P, 16, 64, P, 33, P, 0, None), -2),        # batch > 32
    ((P, 0, 64, P, 1, P, 0, None), -2),          # no rows
    ((P, 16, 32768, P, 1, P, 0, None), -2),      # hidden too large
    ((P, 16, 64, P, 1, P, 5, None), -4),         # bad dtype
    ((ctypes.c_void_p(0x10008), 16, 64, P, 1, P, 0, None), -3),  # misaligned weights
])
def test_gateup_validation(args, status):
    assert tt.lib.tt_mxfp4_gateup_swiglu(*args) == status
    assert tt.lib.tt_last_error().decode()


def test_moe_and_int4_validation():
    L = tt.lib
    assert L.tt_moe_route_topk(P, 1, 32, 9, P, P, None) == -2        # topk > 8
    assert L.tt_moe_route_topk(P, 1, 3, 4, P, P, None) == -2         # topk > n_experts
    assert L.tt_moe_route_topk(P, 1, 300, 4, P, P, None) == -2       # too many experts
    assert L.tt_moe_mxfp4_gateup_swiglu(P, 32, 64, 64, P, 1, None, 4, P, 0, None) == -1
    assert L.tt_moe_mxfp4_down_combine(P, 32, 64, 48, P, 0, P, P, 1, 4, P, 0, None) == -2
    assert L.tt_moe_mxfp4_down_combine(P, 32, 64, 64, P, 3, P, P, 1, 4, P, 0, None) == -4
    assert L.tt_int4_gemv(P, 16, 129, 128, P, 1, P, 0, None) == -2   # odd k
    assert L.tt_int4_gemv(P, 16, 128, 64, P, 1, P, 0, None) == -2    # group != 128
    assert L.tt_mxfp4_gateup_dequantize(P, 8, 64, None, None, None, None, None) == -1


def test_pack_sizes_and_size_errors():
    assert tt.mxfp4_gateup_pack_bytes(11008, 2048) == 1376 * (8 * 2048 + 256 * 4 + 128)
    assert tt.mxfp4_matrix_pack_bytes(2880, 2880) == 180 * (8 * 2880 + 256 * 6 + 128)
    assert tt.int4_pack_bytes(7680, 5120) == 7680 * 5120 // 2 + 7680 * 40 * 4
    with pytest.raises(tt.TTError):
        tt.mxfp4_gateup_pack_bytes(16, 33)
    g, u = workloads.gateup(workloads.TINY)
    small = np.empty(100, np.uint8)
    with pytest.raises(tt.TTError) as e:
        tt.pack_mxfp4_gateup(g, u, 512, 256, out=small)
    assert e.value.status == -5


def test_packers_refuse_short_host_arrays():
    """The packers read their inputs through raw pointers; a short array is
    refused before the call instead of being read past its end."""
    g, u = workloads.gateup(workloads.TINY)
    with pytest.raises(ValueError, match="gate codes"):
        tt.pack_mxfp4_gateup((g[0][:-1], g[1], g[2]), u, 512, 256)
    with pytest.raises(ValueError, match="up ps"):
        tt.pack_mxfp4_gateup(g, (u[0], u[1], u[2][:-1]), 512, 256)
    codes, scales, ps = g
    with pytest.raises(ValueError, match="scales"):
        tt.pack_mxfp4_matrix(codes, scales[:-1], ps, 512, 256)
    fc = np.zeros((8, 64), np.uint8)
    with pytest.raises(ValueError, match="scale"):
        tt.pack_fp8_matrix(fc, np.ones(7, np.float32), 8, 64)
    q, sc, z = tt.quantize_int4_affine(np.ones((4, 256), np.float32))
    with pytest.raises(ValueError, match="z"):
        tt.pack_int4(q, sc, z[:-1], 4, 256)
    # the full-size arrays still pack
    tt.pack_int4(q, sc, z, 4, 256)
    tt.pack_fp8_matrix(fc, np.ones(8, np.float32), 8, 64)


def test_tensors_of_a_call_share_its_device():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4)
    tt._same_device(a, b=torch.zeros(2))
    with pytest.raises(ValueError, match="b is on meta"):
        tt._same_device(a, b=torch.zeros(2, device="meta"))


def _unpack_mx(packed, nrows_tiles, k):
    """Read the documented tiled layout back into canonical arrays (tile row
    order): codes [16T][k/2], scales [16T][k/32], ps [16T]."""
    nb = k // 32
    units = -(-nb // 4)
    qv_last = nb - 4 * (units - 1)
    groups = -(-units // 4)
    scale_off = 256 * nb
    ps_off = scale_off + 256 * groups
    stride = ps_off + 128
    T = nrows_tiles
    codes = np.zeros((16 * T, k // 2), np.uint8)
    scales = np.zeros((16 * T, nb), np.uint8)
    ps = np.zeros(16 * T, np.float32)
    for t in range(T):
        tb = packed[t * stride:(t + 1) * stride]
        for kk in range(units):
            qv = qv_last if kk == units - 1 else 4
            for q in range(qv):
                blk = 4 * kk + q
                for r in range(16):
                    lane = r + 16 * q
                    codes[16 * t + r, 16 * blk:16 * blk + 16] = tb[1024 * kk + 16 * lane:
                                                                   1024 * kk + 16 * lane + 16]
                    scales[16 * t + r, blk] = tb[scale_off + 256 * (kk // 4) + 4 * lane + kk % 4]
        ps[16 * t:16 * t + 16] = tb[ps_off:ps_off + 64].view(np.float32)
    return codes, scales, ps


@pytest.mark.parametrize("n,k", [(40, 256), (16, 2880), (5, 96)])
def test_matrix_pack_follows_documented_layout(n, k):
    c, s, p = workloads.mxfp4_matrix(9, 0, n, k)
    packed = tt.pack_mxfp4_matrix(c, s, p, n, k)
    T = -(-n // 16)
    uc, us, up = _unpack_mx(packed, T, k)
    assert np.array_equal(uc[:n], c) and np.array_equal(us[:n], s) and np.array_equal(up[:n], p)
    assert not uc[n:].any() and np.all(us[n:] == 127)


def test_gateup_pack_interleaves_gate_and_up():
    w = workloads.Workload(9, "t", 160, 20)
    g, u = workloads.gateup(w)
    packed = tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden)
    uc, us, up = _unpack_mx(packed, 3, w.hidden)
    for t in range(3):
        for i in range(8):
            row = 8 * t + i
            if row >= w.inter:
                continue
            assert np.array_equal(uc[16 * t + i], g[0][row])
            assert np.array_equal(uc[16 * t + 8 + i], u[0][row])
            assert np.array_equal(us[16 * t + 8 + i], u[1][row])
            assert up[16 * t + i] == g[2][row] and up[16 * t + 8 + i] == u[2][row]


@pytest.mark.parametrize("n,k", [(64, 5120), (40, 200), (9, 328), (3, 2)])
def test_int4_quantizer_matches_oracle_bit_for_bit(n, k):
    w = workloads.int4_source(2, 0, n, k)
    w[0, : min(128, k)] = 0.0
    q1, s1, z1 = tt.quantize_int4_affine(w)
    q2, s2, z2 = oracle.int4_quantize(w, 128)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2) and np.array_equal(z1, z2)


def test_int4_quantizer_range_error_writes_nothing():
    w = np.array([[-1e6, 1e6]], np.float32)
    with pytest.raises(tt.TTError) as e:
        tt.quantize_int4_affine(w)
    assert e.value.status == -6


def _stored_scale(q, s, z, row, g, k):
    """The scale the packer stores for group g of a row: a zero of the same
    sign when every code of the group equals its zero point and the scale is
    finite, else the scale itself."""
    codes = np.stack([q[row] & 15, q[row] >> 4], axis=1).reshape(-1)[:k]
    grp = codes[128 * g:min(128 * (g + 1), k)].astype(np.float64)
    sv, zv = oracle.f16_value(int(s[row, g])), oracle.f16_value(int(z[row, g]))
    if np.isfinite(sv) and np.all(grp == zv):
        return int(s[row, g]) & 0x8000
    return int(s[row, g])


def test_int4_pack_stores_zero_scale_for_zero_groups():
    """Groups whose codes all equal the zero point get a zero scale of the
    scale's sign; the decoded weights keep their bits."""
    n, k = 4, 300
    w = workloads.int4_source(2, 3, n, k)
    w[0] = 0.0                          # quantizer: s = 1, z = 0, q = 0
    w[1, 128:256] = 0.0
    q, s, z = oracle.int4_quantize(w, 128)
    q[2, 64:128] = 0x99                 # group 1 of row 2: q = z = 9, negative scale
    z[2, 1] = oracle.f16_from_double(9.0)
    s[2, 1] = oracle.f16_from_double(-0.5)
    q[3, 128:150] = 0x55                # partial last group: q = z = 5
    z[3, 2] = oracle.f16_from_double(5.0)
    packed = tt.pack_int4(q, s, z, n, k)
    nq = -(-k // 32)
    sz_off = 256 * nq
    stored = lambda r, g: int(packed[sz_off + 256 * (g // 4) + 16 * r + 4 * (g % 4):][:2]
                              .view(np.uint16)[0])
    for r, g, want in ((0, 0, 0), (0, 2, 0), (1, 1, 0), (2, 1, 0x8000), (3, 2, 0)):
        assert stored(r, g) == want, (r, g, hex(stored(r, g)))
        assert stored(r, g) == _stored_scale(q, s, z, r, g, k)
    assert stored(1, 0) == int(s[1, 0]) != 0


def test_int4_pack_layout():
    n, k = 20, 200
    w = workloads.int4_source(2, 0, n, k)
    w[3, :128] = 0.0
    q, s, z = oracle.int4_quantize(w, 128)
    packed = tt.pack_int4(q, s, z, n, k)
    nq = -(-k // 32)
    units = -(-nq // 4)
    sz_off = 256 * nq
    stride = sz_off + 256 * (-(-units // 4))
    assert packed.size == 2 * stride
    for t in range(2):
        tb = packed[t * stride:(t + 1) * stride]
        for r in range(16):
            row = 16 * t + r
            for kk in range(units):
                v = tb[sz_off + 256 * (kk // 4) + 16 * r + 4 * (kk % 4):][:4].view(np.uint32)[0]
                if row < n:
                    assert v == (_stored_scale(q, s, z, row, kk, k) | (int(z[row, kk]) << 16))
                else:
                    assert v == 0
            for p in range(nq):
                kk, qq = divmod(p, 4)
                got = tb[1024 * kk + 16 * (r + 16 * qq):][:16]
                if row < n:
                    want = np.zeros(16, np.uint8)
                    seg = q[row, 16 * p:16 * p + 16]
                    want[:seg.size] = seg
                    assert np.array_equal(got, want)


def _quant_inputs(n, k, seed):
    gen = np.random.default_rng(seed)
    w = (gen.standard_normal((n, k)) * np.exp2(gen.integers(-20, 20, (n, 1)))).astype(np.float32)
    w[0, :32] = 0.0                                   # all-zero block
    w[1, :8] = [5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 4]  # ties
    w[1, 8] = -0.0
    w[1, 9] = -0.01                                   # rounds to -0
    if n > 2:
        w[2, :2] = [3e38, -1e38]                      # near the fp32 top
    if n > 3:
        w[3, :2] = [1e-40, -2e-41]                    # fp32 subnormals
    return w


@pytest.mark.parametrize("n,k,fit", [(5, 32, True), (37, 256, True), (64, 2048, False),
                                     (3, 2880, True)])
def test_mxfp4_quantizer_matches_oracle_bit_for_bit(n, k, fit):
    w = _quant_inputs(n, k, n + k)
    c1, s1, p1 = tt.quantize_mxfp4(w, fit_postscale=fit)
    c2, s2, p2 = oracle.mxfp4_quantize(w, fit_postscale=fit)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1, s2)
    if fit:
        assert np.array_equal(p1.view(np.uint32), p2.view(np.uint32))
    else:
        assert p1 is None and p2 is None


def test_mxfp4_quantizer_errors_write_nothing():
    w = np.ones((2, 64), np.float32)
    w[1, 40] = np.nan
    codes = np.full((2, 32), 0xAB, np.uint8)
    scales = np.full((2, 2), 0xCD, np.uint8)
    rc = tt.lib.tt_quantize_mxfp4(w.ctypes.data, 2, 64, codes.ctypes.data, scales.ctypes.data,
                                  None)
    assert rc == -6
    assert np.all(codes == 0xAB) and np.all(scales == 0xCD)
    rc = tt.lib.tt_quantize_mxfp4(w.ctypes.data, 2, 48, codes.ctypes.data, scales.ctypes.data,
                                  None)
    assert rc == -2


@pytest.mark.parametrize("n,k", [(13, 200), (8, 128), (20, 300)])
def test_fp8_pack_follows_documented_layout(n, k):
    codes, scale = workloads.fp8_matrix(5, 0, n, k)
    packed = tt.pack_fp8_matrix(codes, scale, n, k)
    units = -(-k // 128)
    stride = 1024 * units + 64
    tiles = -(-n // 8)
    assert packed.size == tiles * stride == tt.fp8_pack_bytes(n, k)
    for t in range(tiles):
        tb = packed[t * stride:(t + 1) * stride]
        sc = tb[1024 * units:1024 * units + 32].view(np.float32)
        for r in range(8):
            row = 8 * t + r
            assert sc[r] == (scale[row] if row < n else 0.0)
            for u in range(units):
                for q in range(8):
                    got = tb[1024 * u + 16 * (r + 8 * q):][:16]
                    k0 = 128 * u + 16 * q
                    want = np.zeros(16, np.uint8)
                    if row < n and k0 < k:
                        seg = codes[row, k0:min(k0 + 16, k)]
                        want[:seg.size] = seg
                    assert np.array_equal(got, want), (t, r, u, q)


def test_fp8_validation():
    P = ctypes.c_void_p(16)
    assert tt.lib.tt_fp8_gemv(P, 8, 100, P, 1, 1, P, 0, None) == -2   # bf16 needs k % 8
    assert tt.lib.tt_fp8_gemv(P, 8, 102, P, 0, 1, P, 0, None) == -2   # fp32 needs k % 4
    assert tt.lib.tt_fp8_gemv(None, 8, 128, P, 0, 1, P, 0, None) == -1
    assert tt.lib.tt_fp8_gemv(P, 8, 128, P, 2, 1, P, 0, None) == -4   # dtype
    assert tt.lib.tt_fp8_gemv(P, 8, 40000, P, 0, 1, P, 0, None) == -2  # k range
    assert tt.lib.tt_fp8_gemv(P, 8, 128, P, 0, 33, P, 0, None) == -2   # batch range
    assert tt.lib.tt_fp8_gemv(ctypes.c_void_p(8), 8, 128, P, 0, 1, P, 0, None) == -3
    assert tt.fp8_pack_bytes(16, 256) == 2 * (2 * 1024 + 64)


def test_attention_validation():
    P = ctypes.c_void_p(16)
    f = tt.lib.tt_gqa_attention_decode
    ok = dict(hq=40, hkv=10, d=128, tcap=512, T=300)
    need = tt.gqa_attention_workspace_bytes(40, 10, 128, 300)
    # hq x chunks x (d + 2) floats; chunks of 32 positions for the split up
    # to T = 2048, of 64 above it and for the one-launch path (at most
    # 256 / d chunks of 64), which still reports the split's size
    assert need == 40 * 10 * 130 * 4
    assert tt.gqa_attention_workspace_bytes(40, 10, 128, 2048) == 40 * 64 * 130 * 4
    assert tt.gqa_attention_workspace_bytes(40, 10, 128, 2049) == 40 * 33 * 130 * 4
    assert tt.gqa_attention_workspace_bytes(40, 10, 128, 100) == 40 * 2 * 130 * 4
    assert tt.gqa_attention_workspace_bytes(64, 8, 64, 256) == 64 * 4 * 66 * 4
    assert tt.gqa_attention_workspace_bytes(64, 8, 64, 257) == 64 * 9 * 66 * 4
    def call(hq=40, hkv=10, d=128, tcap=512, T=300, ws=need, dt=0, ptr=P):
        return f(ptr, P, P, hq, hkv, d, tcap, T, 0.1, P, dt, P, ws, None)
    assert call(hq=30) == -2              # not a multiple
    assert call(hq=48, hkv=4) == -2       # group 12
    assert call(d=96) == -2
    assert call(T=600) == -2              # T > tcap
    assert call(ws=need - 1) == -5
    assert call(dt=3) == -4
    assert call(ptr=None) == -1
    assert call(ptr=ctypes.c_void_p(8)) == -3
