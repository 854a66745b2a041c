"""The device calls under HIP graph capture: every replay must reproduce
the eager result, with eager work and synchronisations between replays; the
captured dense decode layer is also checked stage by stage against the
oracle."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import workloads
import oracle
from _parity import assert_parity, dev_bf16, dev_u8, gemv_tol, h_tol, to_np

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replays_match_eager(dev):
    w = workloads.Workload(9, "graph", 2880, 1024, n_experts=6, topk=4)
    g, u = workloads.gateup(w)
    gu = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    gb = workloads.expert_bank(w, 0, "gate")
    ub = workloads.expert_bank(w, 0, "up")
    db = workloads.expert_bank(w, 0, "down")
    gs = tt.mxfp4_gateup_pack_bytes(w.inter, w.hidden)
    ds = tt.mxfp4_matrix_pack_bytes(w.hidden, w.inter)
    bank = np.empty(6 * gs, np.uint8)
    down = np.empty(6 * ds, np.uint8)
    for e in range(6):
        tt.pack_mxfp4_gateup((gb[0][e], gb[1][e], gb[2][e]), (ub[0][e], ub[1][e], ub[2][e]),
                             w.inter, w.hidden, out=bank[e * gs:(e + 1) * gs])
        tt.pack_mxfp4_matrix(db[0][e], db[1][e], db[2][e], w.hidden, w.inter,
                             out=down[e * ds:(e + 1) * ds])
    bank, down = dev_u8(bank, dev), dev_u8(down, dev)
    wq = workloads.int4_source(2, 0, 384, w.hidden)
    q4 = dev_u8(tt.pack_int4(*tt.quantize_int4_affine(wq), 384, w.hidden), dev)

    x1 = dev_bf16(workloads.activations(9, 0, 1, w.hidden), dev)
    x8 = dev_bf16(workloads.activations(9, 1, 8, w.hidden), dev)
    lg = dev_bf16(workloads.router_logits(9, 0, 1, 6), dev)
    outs = dict(h1=torch.empty((1, w.inter), device=dev), h8=torch.empty((8, w.inter), device=dev),
                ids=torch.empty((1, 4), dtype=torch.int32, device=dev),
                wt=torch.empty((1, 4), device=dev),
                he=torch.empty((1, 4, w.inter), dtype=torch.bfloat16, device=dev),
                y=torch.empty((1, w.hidden), device=dev), q=torch.empty((1, 384), device=dev))

    def step():
        tt.mxfp4_gateup_swiglu(gu, w.inter, w.hidden, x1, out=outs["h1"])
        tt.mxfp4_gateup_swiglu(gu, w.inter, w.hidden, x8, out=outs["h8"])
        tt.moe_route_topk(lg, 4, ids=outs["ids"], w=outs["wt"])
        tt.moe_mxfp4_gateup_swiglu(bank, 6, w.inter, w.hidden, x1, outs["ids"], out=outs["he"])
        tt.moe_mxfp4_down_combine(down, 6, w.hidden, w.inter, outs["he"], outs["ids"],
                                  outs["wt"], out=outs["y"])
        tt.int4_gemv(q4, 384, w.hidden, x1, out=outs["q"])

    graph = _capture(step)
    gen = np.random.default_rng(0)
    for rep in range(4):
        # new inputs in place (eager work between replays)
        x1.copy_(dev_bf16(workloads.bf16_bits(gen.standard_normal((1, w.hidden))
                                              .astype(np.float32)), dev))
        lg.copy_(dev_bf16(workloads.bf16_bits(gen.standard_normal((1, 6))
                                              .astype(np.float32)), dev))
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        eager = {k: v.clone() for k, v in outs.items()}
        for v in outs.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], eager[k]), (rep, k)


@pytest.mark.parametrize("shape", ["small", "phi4"])
def test_one_graph_per_dense_decode_layer(dev, shape):
    """A whole dense decode layer captured as one graph -- INT4 QKV (bf16
    out) -> GQA attention on the q heads -> INT4 O (bf16 out) -> MXFP4
    gate/up SwiGLU -> FP8 down.  Every replay equals the eager chain, and
    every stage of the last replay matches the oracle fed the device's own
    output of the stage before (so each stage is held to its own bound).
    "phi4" is the Phi-4-shaped layer (40 / 10 heads of 128, hidden 5120,
    inter 17920, 1024 cached positions)."""
    if shape == "small":
        hq, hkv, d, T, hidden, inter = 8, 2, 128, 300, 1024, 768
    else:
        hq, hkv, d, T, hidden, inter = 40, 10, 128, 1024, 5120, 17920
    nq = (hq + 2 * hkv) * d
    gen = np.random.default_rng(5)
    q1 = tt.quantize_int4_affine(workloads.int4_source(3, 0, nq, hidden))
    q2 = tt.quantize_int4_affine(workloads.int4_source(3, 1, hidden, hq * d))
    qkv = dev_u8(tt.pack_int4(*q1, nq, hidden), dev)
    o4 = dev_u8(tt.pack_int4(*q2, hidden, hq * d), dev)
    w = workloads.Workload(3, "layer", hidden, inter)
    g, u = workloads.gateup(w)
    gu = dev_u8(tt.pack_mxfp4_gateup(g, u, inter, hidden), dev)
    dc, dsc = workloads.fp8_matrix(3, 0, hidden, inter)
    dn = dev_u8(tt.pack_fp8_matrix(dc, dsc, hidden, inter), dev)
    kh = workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32))
    vh = workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32))
    kc, vc = dev_bf16(kh, dev), dev_bf16(vh, dev)
    x = dev_bf16(workloads.activations(3, 0, 1, hidden), dev)
    ws = torch.empty(tt.gqa_attention_workspace_bytes(hq, hkv, d, T), dtype=torch.uint8,
                     device=dev)
    outs = dict(qkv=torch.empty((1, nq), dtype=torch.bfloat16, device=dev),
                att=torch.empty((hq, d), dtype=torch.bfloat16, device=dev),
                o=torch.empty((1, hidden), dtype=torch.bfloat16, device=dev),
                h=torch.empty((1, inter), device=dev),
                y=torch.empty((1, hidden), device=dev))
    scale = d ** -0.5

    def step():
        tt.int4_gemv(qkv, nq, hidden, x, out=outs["qkv"])
        q = outs["qkv"][0, :hq * d]
        tt.gqa_attention_decode(q, kc, vc, hq, hkv, d, T, scale, out=outs["att"],
                                workspace=ws)
        tt.int4_gemv(o4, hidden, hq * d, outs["att"].view(1, hq * d), out=outs["o"])
        tt.mxfp4_gateup_swiglu(gu, inter, hidden, outs["o"], out=outs["h"])
        tt.fp8_gemv(dn, hidden, inter, outs["h"], out=outs["y"])

    graph = _capture(step)
    for rep in range(3):
        x.copy_(dev_bf16(workloads.bf16_bits(gen.standard_normal((1, hidden))
                                             .astype(np.float32)), dev))
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        eager = {k: v.clone() for k, v in outs.items()}
        for v in outs.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], eager[k]), (rep, k)
        assert torch.isfinite(outs["y"]).all()

    # each stage of the last replay against the oracle, fed the device's own
    # input to that stage
    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    x_b = bits(x)
    ref, S = oracle.int4_gemv(*q1, nq, hidden, 128, x_b)
    assert_parity(to_np(outs["qkv"]), ref, gemv_tol(S, ref, bf16=True), f"{shape} layer: QKV")
    q_b = bits(outs["qkv"])[:, :hq * d].reshape(hq, d)
    ref, A, Smax = oracle.gqa_attention(q_b, kh, vh, hq, hkv, d, T, T, scale)
    tol = (2e-3 + 4e-5 * Smax[:, None]) * A + 2.0 ** -8 * np.abs(ref)
    assert_parity(to_np(outs["att"]), ref, tol, f"{shape} layer: attention")
    att_b = bits(outs["att"]).reshape(1, hq * d)
    ref, S = oracle.int4_gemv(*q2, hidden, hq * d, 128, att_b)
    assert_parity(to_np(outs["o"]), ref, gemv_tol(S, ref, bf16=True), f"{shape} layer: O")
    o_b = bits(outs["o"])
    ref = oracle.mxfp4_gateup_swiglu(g, u, inter, hidden, o_b, parallel=True)
    assert_parity(to_np(outs["h"]), ref["h"], h_tol(ref), f"{shape} layer: gate/up SwiGLU")
    h_f = outs["h"].cpu().numpy()
    ref, S = oracle.fp8_gemv(dc, dsc, hidden, inter, h_f)
    assert_parity(to_np(outs["y"]), ref, gemv_tol(S, ref), f"{shape} layer: FP8 down")
