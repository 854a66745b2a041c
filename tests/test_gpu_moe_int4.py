"""GPU parity of the routed-expert stages and the INT4 matvec against the CPU
oracle, through the C ABI.  The routed-expert tests hold the gpt-oss-20b-shaped
config's whole bank (32 experts, hidden 2880, inter 2880, top-4) on the
device and route over all 32 logits."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import oracle
import workloads
from _parity import (assert_parity, cosine, dev_bf16, dev_u8, gemv_tol, guarded, h_tol,
                     to_np)

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
    """The gpt-oss-20b-shaped config's whole expert bank on the device."""
    w = workloads.GPTOSS
    n_exp = w.n_experts
    gb = workloads.expert_bank(w, 0, "gate")
    ub = workloads.expert_bank(w, 0, "up")
    db = workloads.expert_bank(w, 0, "down")
    return dict(w=w, n_exp=n_exp, gb=gb, ub=ub, db=db,
                gu=dev_u8(_bank_pack(gb, ub, n_exp, w.inter, w.hidden), dev),
                dn=dev_u8(_down_pack(db, n_exp, w.hidden, w.inter), dev))


def _boundary_ties(lg, topk):
    """Plant ties where they decide the routing: the (topk+1)-th largest
    logit of every token made equal to the topk-th (the lower expert index
    must win the last slot), and the second largest equal to the largest."""
    lg = lg.copy()
    for b in range(lg.shape[0]):
        order = np.argsort(-workloads.bf16_to_f32(lg[b]), kind="stable")
        lg[b, order[topk]] = lg[b, order[topk - 1]]
        lg[b, order[1]] = lg[b, order[0]]
    return lg


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("batch", [1, 3])
@pytest.mark.parametrize("h_dtype", [torch.float32, torch.bfloat16])
def test_moe_layer_stages(dev, gptoss, fused, batch, h_dtype):
    """The config's layer stage by stage against the oracle: routing over 32
    logits (separate call, or fused into the expert gate/up as the benchmark
    runs it), expert gate/up SwiGLU, then down + combine on the device's own
    h and routing weights.  Batch 3 carries ties at the selection boundary."""
    w, n_exp = gptoss["w"], gptoss["n_exp"]
    lg = workloads.router_logits(w.wid, 17 + batch, batch, n_exp)
    if batch > 1:
        lg = _boundary_ties(lg, w.topk)
    x = workloads.activations(w.wid, 0, batch, w.hidden)
    xd, lgd = dev_bf16(x, dev), dev_bf16(lg, dev)
    h, hcheck = guarded((batch, w.topk, w.inter), h_dtype, dev)
    if fused:
        _, ids, wt = tt.moe_mxfp4_route_gateup_swiglu(gptoss["gu"], n_exp, w.inter, w.hidden,
                                                      xd, lgd, w.topk, out=h)
    else:
        ids, wt = tt.moe_route_topk(lgd, w.topk)
        tt.moe_mxfp4_gateup_swiglu(gptoss["gu"], n_exp, w.inter, w.hidden, xd, ids, out=h)
    y, ycheck = guarded((batch, w.hidden), torch.float32, dev)
    tt.moe_mxfp4_down_combine(gptoss["dn"], n_exp, w.hidden, w.inter, h, ids, wt, out=y)
    torch.cuda.synchronize()
    hcheck()
    ycheck()
    rid, rw = oracle.moe_route_topk(lg, w.topk)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(wt.cpu().numpy(), rw, rtol=2e-6, atol=0)
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
                w.inter, w.hidden, x[b], parallel=True)
            gr[b, j], ur[b, j] = o["g"][0], o["u"][0]
    ref = dict(h=hr, Sg=Sg, Su=Su, g=gr, u=ur)
    bf = h_dtype == torch.bfloat16
    tag = f"{'fused' if fused else 'separate'} b{batch} {h_dtype}"
    assert_parity(to_np(h), hr, h_tol(ref, bf16=bf), f"moe gate/up {tag}")
    # stage 2: down + combine on the device's own h and routing weights
    hg = to_np(h)
    yr, S = oracle.moe_down_combine(gptoss["db"], n_exp, w.hidden, w.inter, hg, rid,
                                    wt.cpu().numpy().astype(np.float64))
    assert_parity(to_np(y), yr, gemv_tol(S, yr), f"moe down+combine {tag}")
    # end to end against the all-oracle pipeline
    ye, _ = oracle.moe_down_combine(gptoss["db"], n_exp, w.hidden, w.inter, hr, rid, rw)
    c = cosine(to_np(y), ye)
    print(f"moe end-to-end cosine {tag}: {c:.9f}")
    assert c >= 0.99999


@pytest.mark.parametrize("batch", [1, 3])
def test_fused_route_gateup_equals_separate_calls(dev, gptoss, batch):
    w, n_exp = gptoss["w"], gptoss["n_exp"]
    xd = dev_bf16(workloads.activations(w.wid, 2, batch, w.hidden), dev)
    for step in range(4):
        lg = workloads.router_logits(w.wid, 40 + step, batch, n_exp)
        if step == 2:
            lg[:, 1::2] = lg[:, 0::2]          # planted ties
        if step == 3:
            lg = _boundary_ties(lg, w.topk)
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


def _nan_bank(w, which, plant):
    """A canonical bank with E8M0 0xFF planted at (expert, row, block)."""
    bank = workloads.expert_bank(w, 0, which)
    scales = bank[1].copy()
    for e, r, blk in plant:
        scales[e, r, blk] = 0xFF
    return bank[0], scales, bank[2]


@pytest.mark.parametrize("h_dtype", [torch.float32, torch.bfloat16])
def test_moe_nan_scale_blocks(dev, h_dtype):
    """E8M0 0xFF blocks in the routed gate/up (separate and fused routing)
    and in the down projection: NaN exactly where the oracle has it."""
    n_exp, topk = 6, 3
    w = workloads.Workload(9, "nanmoe", 512, 384, n_experts=n_exp, topk=topk)
    nb_h, nb_i = w.hidden // 32, w.inter // 32
    gb = _nan_bank(w, "gate", [(0, 3, 0), (2, 100, nb_h - 1), (5, 383, 7)])
    ub = _nan_bank(w, "up", [(0, 7, 2), (2, 0, 0), (4, 200, nb_h - 1)])
    db = _nan_bank(w, "down", [(1, 5, 0), (3, 511, nb_i - 1), (5, 64, 4)])
    gu = dev_u8(_bank_pack(gb, ub, n_exp, w.inter, w.hidden), dev)
    dn = dev_u8(_down_pack(db, n_exp, w.hidden, w.inter), dev)
    x = workloads.activations(w.wid, 0, 2, w.hidden)
    xd = dev_bf16(x, dev)
    ids_np = np.array([[0, 2, 5], [4, 1, 3]], np.int32)
    ids = torch.from_numpy(ids_np).to(dev)
    h = tt.moe_mxfp4_gateup_swiglu(gu, n_exp, w.inter, w.hidden, xd, ids, out_dtype=h_dtype)
    hr, Sg, Su = oracle.moe_gateup_swiglu(gb, ub, n_exp, w.inter, w.hidden, x, ids_np)
    gr, ur = np.empty_like(hr), np.empty_like(hr)
    for b in range(2):
        for j in range(topk):
            e = ids_np[b, j]
            o = oracle.mxfp4_gateup_swiglu((gb[0][e], gb[1][e], gb[2][e]),
                                           (ub[0][e], ub[1][e], ub[2][e]), w.inter, w.hidden, x[b])
            gr[b, j], ur[b, j] = o["g"][0], o["u"][0]
    assert np.isnan(hr).any()
    ref = dict(h=hr, Sg=Sg, Su=Su, g=gr, u=ur)
    assert_parity(to_np(h), hr, h_tol(ref, bf16=h_dtype == torch.bfloat16),
                  f"moe gate/up NaN blocks {h_dtype}")
    # fused routing: logits that select experts 0, 2, 5 for token 0
    lg = np.zeros((1, n_exp), np.float32)
    lg[0, [0, 2, 5]] = [3.0, 2.0, 1.0]
    hf, idf, _ = tt.moe_mxfp4_route_gateup_swiglu(gu, n_exp, w.inter, w.hidden, xd[:1],
                                                  dev_bf16(workloads.bf16_bits(lg), dev), topk,
                                                  out_dtype=h_dtype)
    assert np.array_equal(idf.cpu().numpy(), ids_np[:1])
    assert_parity(to_np(hf), hr[:1], h_tol({k: v[:1] for k, v in ref.items()},
                                           bf16=h_dtype == torch.bfloat16),
                  f"moe fused gate/up NaN blocks {h_dtype}")
    # down: finite h, NaN blocks in experts 1, 3 and 5
    gen = np.random.default_rng(8)
    hin = gen.standard_normal((2, topk, w.inter)).astype(np.float32)
    if h_dtype == torch.bfloat16:
        hin = workloads.bf16_to_f32(workloads.bf16_bits(hin))
    wt = gen.uniform(0.1, 1.0, (2, topk)).astype(np.float32)
    for dids in (np.array([[1, 0, 2], [4, 2, 0]], np.int32), ids_np):
        y = tt.moe_mxfp4_down_combine(dn, n_exp, w.hidden, w.inter,
                                      torch.from_numpy(hin).to(dev).to(h_dtype),
                                      torch.from_numpy(dids).to(dev), torch.from_numpy(wt).to(dev))
        yr, S = oracle.moe_down_combine(db, n_exp, w.hidden, w.inter, hin, dids,
                                        wt.astype(np.float64))
        assert_parity(to_np(y), yr, gemv_tol(S, yr), f"moe down NaN blocks {h_dtype} {dids[0]}")


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
    y, check = guarded((2, hidden), torch.float32, dev)
    tt.moe_mxfp4_down_combine(dn, n_exp, w.hidden, w.inter, hd, torch.from_numpy(ids).to(dev),
                              torch.from_numpy(wt).to(dev), out=y)
    check()
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
    """Every row, including the Phi-4-shaped QKV (7680 x 5120) and O
    (5120 x 5120) projections."""
    q, s, z, packed, x = _int4_case(dev, n, k, batch)
    y, check = guarded((batch, n), torch.float32, dev)
    tt.int4_gemv(packed, n, k, dev_bf16(x, dev), out=y)
    check()
    yr, S = oracle.int4_gemv(q, s, z, n, k, 128, x)
    assert_parity(to_np(y), yr, gemv_tol(S, yr), f"int4 n{n} k{k} b{batch}")


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_int4_zero_groups_are_exact(dev, batch):
    """Groups whose codes all equal their zero point contribute exactly 0:
    the quantizer's all-zero groups (s = 1, z = 0, q = 0), all-zero rows,
    and hand-made groups with q = z = 7 under a random scale.  Rows made only
    of such groups must come out exactly 0.0; the rest match the oracle."""
    n, k = 64, 1000
    wsrc = workloads.int4_source(2, 5, n, k)
    wsrc[0] = 0.0                       # an all-zero row
    wsrc[1, :128] = 0.0                 # all-zero first group
    wsrc[2, 896:] = 0.0                 # all-zero partial last group (104 elements)
    wsrc[3:6, 128:640] = 0.0            # several zero groups in the middle
    q, s, z = oracle.int4_quantize(wsrc, 128)
    G = -(-k // 128)
    for r in (6, 7):                    # rows of groups with q = z = 7
        q[r] = 0x77
        z[r] = oracle.f16_from_double(7.0)
        s[r] = [oracle.f16_from_double(float(v)) for v in
                np.random.default_rng(r).uniform(1e-3, 1e-1, G)]
    packed = dev_u8(tt.pack_int4(q, s, z, n, k), dev)
    x = workloads.activations(2, 9, batch, k, tensor=workloads.T_OX)
    y = to_np(tt.int4_gemv(packed, n, k, dev_bf16(x, dev)))
    yr, S = oracle.int4_gemv(q, s, z, n, k, 128, x)
    for r in (0, 6, 7):
        assert np.all(yr[:, r] == 0.0)
        assert np.all(y[:, r] == 0.0), (r, y[:, r])
    assert_parity(y, yr, gemv_tol(S, yr), f"int4 zero groups b{batch}")


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
