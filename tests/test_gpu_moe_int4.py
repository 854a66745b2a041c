"""GPU parity of the routed-expert stages and the INT4 matvec against the CPU
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import (assert_parity, cosine, dev_bf16, dev_u8, gemv_tol, h_tol, to_np)

pytestmark = pytest.mark.gpu


def _bank_pack(bank_g, bank_u, n_exp, inter, hidden):
    stride = tt.mxfp4_gateup_pack_bytes(inter, hidden)
    out = np.empty(n_exp * stride, np.uint8)
    for e in range(n_exp):
        tt.pack_mxfp4_gateup((bank_g[0][e], bank_g[1][e], bank_g[2][e]),
                             (bank_u[0][e], bank_u[1][e], bank_u[2][e]), inter, hidden,
                             out=out[e * stride:(e + 1) * stride])
    return out


def _down_pack(bank_d, n_exp, hidden, inter):
    stride = tt.mxfp4_matrix_pack_bytes(hidden, inter)
    out = np.empty(n_exp * stride, np.uint8)
    for e in range(n_exp):
        tt.pack_mxfp4_matrix(bank_d[0][e], bank_d[1][e], bank_d[2][e], hidden, inter,
                             out=out[e * stride:(e + 1) * stride])
    return out


# ---- routing ----------------------------------------------------------------

@pytest.mark.parametrize("n_exp,topk,batch", [(32, 4, 1), (32, 4, 32), (256, 8, 5), (8, 8, 3),
                                              (100, 3, 7)])
def test_route_topk(dev, n_exp, topk, batch):
    lg = workloads.router_logits(3, n_exp + topk, batch, n_exp)
    lg2 = lg.copy()
    lg2[:, 1::3] = lg2[:, 0::3][:, : lg2[:, 1::3].shape[1]]   # planted ties
    for logits in (lg, lg2):
        ids, w = tt.moe_route_topk(dev_bf16(logits, dev), topk)
        rid, rw = oracle.moe_route_topk(logits, topk)
        assert np.array_equal(ids.cpu().numpy(), rid)
        assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=0)


# ---- expert gate/up and down --------------------------------------------------

@pytest.fixture(scope="module")
def gptoss(dev):
    w = workloads.GPTOSS
    n_exp = 8   # experts held on the device for the test; ids are remapped below
    gb = workloads.expert_bank(w, 0, "gate", n_experts=n_exp)
    ub = workloads.expert_bank(w, 0, "up", n_experts=n_exp)
    db = workloads.expert_bank(w, 0, "down", n_experts=n_exp)
    return dict(w=w, n_exp=n_exp, gb=gb, ub=ub, db=db,
                gu=dev_u8(_bank_pack(gb, ub, n_exp, w.inter, w.hidden), dev),
                dn=dev_u8(_down_pack(db, n_exp, w.hidden, w.inter), dev))


@pytest.mark.parametrize("batch", [1, 3])
@pytest.mark.parametrize("h_dtype", [torch.float32, torch.bfloat16])
def test_moe_layer_stages(dev, gptoss, batch, h_dtype):
    w, n_exp = gptoss["w"], gptoss["n_exp"]
    lg = workloads.router_logits(w.wid, 17 + batch, batch, n_exp)
    x = workloads.activations(w.wid, 0, batch, w.hidden)
    ids, wt = tt.moe_route_topk(dev_bf16(lg, dev), w.topk)
    h = tt.moe_mxfp4_gateup_swiglu(gptoss["gu"], n_exp, w.inter, w.hidden, dev_bf16(x, dev),
                                   ids, out_dtype=h_dtype)
    y = tt.moe_mxfp4_down_combine(gptoss["dn"], n_exp, w.hidden, w.inter, h, ids, wt)
    torch.cuda.synchronize()
    rid, rw = oracle.moe_route_topk(lg, w.topk)
    assert np.array_equal(ids.cpu().numpy(), rid)
    # stage 1: expert gate/up against the oracle
    hr, Sg, Su = oracle.moe_gateup_swiglu(gptoss["gb"], gptoss["ub"], n_exp, w.inter, w.hidden,
                                          x, rid)
    gr = np.empty_like(hr)
    ur = np.empty_like(hr)
    for b in range(batch):
        for j in range(w.topk):
            e = rid[b, j]
            o = oracle.mxfp4_gateup_swiglu(
                (gptoss["gb"][0][e], gptoss["gb"][1][e], gptoss["gb"][2][e]),
                (gptoss["ub"][0][e], gptoss["ub"][1][e], gptoss["ub"][2][e]),
                w.inter, w.hidden, x[b])
            gr[b, j], ur[b, j] = o["g"][0], o["u"][0]
    ref = dict(h=hr, Sg=Sg, Su=Su, g=gr, u=ur)
    bf = h_dtype == torch.bfloat16
    assert_parity(to_np(h), hr, h_tol(ref, bf16=bf), f"moe gate/up b{batch} {h_dtype}")
    # stage 2: down + combine on the device's own h and routing weights
    hg = to_np(h)
    yr, S = oracle.moe_down_combine(gptoss["db"], n_exp, w.hidden, w.inter, hg, rid,
                                    wt.cpu().numpy().astype(np.float64))
    assert_parity(to_np(y), yr, gemv_tol(S, yr), f"moe down+combine b{batch} {h_dtype}")
    # end to end against the all-oracle pipeline
    ye, _ = oracle.moe_down_combine(gptoss["db"], n_exp, w.hidden, w.inter, hr, rid, rw)
    c = cosine(to_np(y), ye)
    print(f"moe end-to-end cosine b{batch} {h_dtype}: {c:.9f}")
    assert c >= 0.99999


@pytest.mark.parametrize("batch", [1, 3])
def test_fused_route_gateup_equals_separate_calls(dev, gptoss, batch):
    w, n_exp = gptoss["w"], gptoss["n_exp"]
    xd = dev_bf16(workloads.activations(w.wid, 2, batch, w.hidden), dev)
    for step in range(3):
        lg = workloads.router_logits(w.wid, 40 + step, batch, n_exp)
        if step == 2:
            lg[:, 1::2] = lg[:, 0::2]          # planted ties
        lgd = dev_bf16(lg, dev)
        ids, wt = tt.moe_route_topk(lgd, w.topk)
        h = tt.moe_mxfp4_gateup_swiglu(gptoss["gu"], n_exp, w.inter, w.hidden, xd, ids)
        hf, idf, wf = tt.moe_mxfp4_route_gateup_swiglu(gptoss["gu"], n_exp, w.inter, w.hidden,
                                                       xd, lgd, w.topk)
        assert torch.equal(idf, ids) and torch.equal(wf, wt) and torch.equal(hf, h)
        rid, _ = oracle.moe_route_topk(lg, w.topk)
        assert np.array_equal(idf.cpu().numpy(), rid)


def test_moe_single_expert_equals_dense(dev, gptoss):
    w = gptoss["w"]
    x = workloads.activations(w.wid, 5, 1, w.hidden)
    xd = dev_bf16(x, dev)
    e = 6
    ids = torch.tensor([[e]], dtype=torch.int32, device=dev)
    h = tt.moe_mxfp4_gateup_swiglu(gptoss["gu"], gptoss["n_exp"], w.inter, w.hidden, xd, ids)
    stride = tt.mxfp4_gateup_pack_bytes(w.inter, w.hidden)
    hd = tt.mxfp4_gateup_swiglu(gptoss["gu"][e * stride:(e + 1) * stride], w.inter, w.hidden, xd)
    assert torch.equal(h[:, 0], hd)


def test_moe_bad_ids_give_nan_rows(dev, gptoss):
    w = gptoss["w"]
    x = dev_bf16(workloads.activations(w.wid, 0, 1, w.hidden), dev)
    ids = torch.tensor([[1, -1, gptoss["n_exp"], 2]], dtype=torch.int32, device=dev)
    wt = torch.full((1, 4), 0.25, dtype=torch.float32, device=dev)
    h = tt.moe_mxfp4_gateup_swiglu(gptoss["gu"], gptoss["n_exp"], w.inter, w.hidden, x, ids)
    hn = to_np(h)
    assert np.all(np.isfinite(hn[0, 0])) and np.all(np.isfinite(hn[0, 3]))
    assert np.all(np.isnan(hn[0, 1])) and np.all(np.isnan(hn[0, 2]))
    y = tt.moe_mxfp4_down_combine(gptoss["dn"], gptoss["n_exp"], w.hidden, w.inter,
                                  torch.nan_to_num(h), ids, wt)
    assert np.all(np.isnan(to_np(y)))


@pytest.mark.parametrize("hidden,inter,topk,h_bf16", [(96, 160, 3, False), (96, 160, 3, True),
                                                      (40, 2048, 8, True), (48, 4096, 8, False),
                                                      (33, 8192, 5, True)])
def test_moe_down_ragged(dev, hidden, inter, topk, h_bf16):
    """hidden not a multiple of 16, partial units, several slot rounds."""
    n_exp = 9
    w = workloads.Workload(9, "rag", hidden, inter, n_experts=n_exp, topk=topk)
    db = workloads.expert_bank(w, 0, "down")
    dn = dev_u8(_down_pack(db, n_exp, w.hidden, w.inter), dev)
    gen = np.random.default_rng(inter + topk)
    h = gen.standard_normal((2, topk, w.inter)).astype(np.float32)
    if h_bf16:
        h = workloads.bf16_to_f32(workloads.bf16_bits(h))
    ids = gen.integers(0, n_exp, (2, topk)).astype(np.int32)
    wt = gen.uniform(0.05, 1.0, (2, topk)).astype(np.float32)
    hd = torch.from_numpy(h).to(dev)
    if h_bf16:
        hd = hd.to(torch.bfloat16)
    y = tt.moe_mxfp4_down_combine(dn, n_exp, w.hidden, w.inter, hd,
                                  torch.from_numpy(ids).to(dev), torch.from_numpy(wt).to(dev))
    yr, S = oracle.moe_down_combine(db, n_exp, w.hidden, w.inter, h, ids, wt.astype(np.float64))
    assert_parity(to_np(y), yr, gemv_tol(S, yr), f"moe down h{hidden} i{inter} k{topk}")


def test_moe_down_wide_range_bf16_h(dev):
    """bf16 h spread over 2^52 within every block (the two-part E4M3 split of
    the scaled-MFMA down kernel): parity at the usual bar."""
    n_exp, topk = 6, 4
    w = workloads.Workload(9, "widedn", 512, 2880, n_experts=n_exp, topk=topk)
    db = workloads.expert_bank(w, 0, "down")
    dn = dev_u8(_down_pack(db, n_exp, w.hidden, w.inter), dev)
    gen = np.random.default_rng(515)
    mag = np.exp2(gen.uniform(-40, 12, (1, topk, w.inter)))
    h = (np.where(gen.random(mag.shape) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    h = workloads.bf16_to_f32(workloads.bf16_bits(h))
    ids = np.array([[0, 5, 2, 3]], np.int32)
    wt = gen.uniform(0.05, 1.0, (1, topk)).astype(np.float32)
    y = tt.moe_mxfp4_down_combine(dn, n_exp, w.hidden, w.inter,
                                  torch.from_numpy(h).to(dev).to(torch.bfloat16),
                                  torch.from_numpy(ids).to(dev), torch.from_numpy(wt).to(dev))
    yr, S = oracle.moe_down_combine(db, n_exp, w.hidden, w.inter, h, ids, wt.astype(np.float64))
    assert_parity(to_np(y), yr, gemv_tol(S, yr), "moe down wide-range bf16 h")


# ---- INT4 ----------------------------------------------------------------------

def _int4_case(dev, n, k, batch, layer=0, tensor=workloads.T_INT4W):
    wsrc = workloads.int4_source(2, layer, n, k, tensor)
    q, s, z = oracle.int4_quantize(wsrc, 128)
    packed = dev_u8(tt.pack_int4(q, s, z, n, k), dev)
    x = workloads.activations(2, layer, batch, k, tensor=workloads.T_OX)
    return q, s, z, packed, x


@pytest.mark.parametrize("n,k,batch", [(7680, 5120, 1), (5120, 5120, 1), (100, 200, 1),
                                       (48, 328, 3), (33, 5120, 8), (16, 2, 1), (40, 130, 32),
                                       (64, 16384, 1), (40, 16384, 3), (24, 1002, 2),
                                       (72, 640, 5), (16, 4096, 6), (8, 256, 31)])
def test_int4_gemv(dev, n, k, batch):
    q, s, z, packed, x = _int4_case(dev, n, k, batch)
    y = tt.int4_gemv(packed, n, k, dev_bf16(x, dev))
    torch.cuda.synchronize()
    rows = None
    got = to_np(y)
    if n > 2048:
        rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                         np.random.default_rng(n).choice(n, 400, replace=False)]))
        got = got[:, rows]
    yr, S = oracle.int4_gemv(q, s, z, n, k, 128, x, rows=rows)
    assert_parity(got, yr, gemv_tol(S, yr), f"int4 n{n} k{k} b{batch}")


@pytest.mark.parametrize("k", [512, 5120])
def test_int4_gemv_unaligned_x(dev, k):
    """x two bytes past a 16-byte boundary takes the element-load instantiation."""
    n = 48
    q, s, z, packed, x = _int4_case(dev, n, k, 1, layer=3)
    xb = dev_bf16(x, dev).reshape(-1)
    buf = torch.zeros(k + 8, dtype=xb.dtype, device=dev)
    buf[1:k + 1] = xb
    xv = buf[1:k + 1].view(1, k)
    assert xv.data_ptr() % 16 == 2
    got = to_np(tt.int4_gemv(packed, n, k, xv))
    yr, S = oracle.int4_gemv(q, s, z, n, k, 128, x)
    assert_parity(got, yr, gemv_tol(S, yr), f"int4 unaligned x k{k}")


def test_int4_dequantize_bit_exact(dev):
    for n, k in ((40, 200), (17, 5120)):
        q, s, z, packed, _ = _int4_case(dev, n, k, 1)
        got = tt.int4_dequantize(packed, n, k).cpu().numpy()
        ref = oracle.int4_dequantize(q, s, z, n, k, 128)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_int4_one_hot_columns(dev):
    n, k = 64, 384
    q, s, z, packed, _ = _int4_case(dev, n, k, 1)
    deq = oracle.int4_dequantize(q, s, z, n, k, 128)
    for j in (0, 127, 128, 383):
        x = np.zeros((1, k), np.uint16)
        x[0, j] = 0x3F80
        y = to_np(tt.int4_gemv(packed, n, k, dev_bf16(x, dev)))
        assert np.array_equal(y[0], deq[:, j].astype(np.float64)), j
