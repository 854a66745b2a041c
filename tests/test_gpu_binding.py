"""The Python binding refuses buffers the call would overrun, before any
launch: outputs shorter than batch x rows, packed weights (or expert banks)
shorter than their packed size, activations that are not whole rows, and an
h of the wrong shape.  The library itself sees only pointers, so these
checks are what keeps a short buffer from becoming an out-of-bounds device
access."""
import numpy as np
import pytest
import torch

import bit_weight_only_mxfp4_amd as tt
import workloads
from _parity import dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def test_short_buffers_are_refused(dev):
    w = workloads.Workload(9, "sizes", 256, 64, n_experts=3, topk=2)
    g, u = workloads.gateup(w)
    gu = dev_u8(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden), dev)
    x = dev_bf16(workloads.activations(9, 0, 2, w.hidden), dev)
    with pytest.raises(ValueError):                      # out too short
        tt.mxfp4_gateup_swiglu(gu, w.inter, w.hidden, x,
                               out=torch.empty((1, w.inter), device=dev))
    with pytest.raises(ValueError):                      # pack too short
        tt.mxfp4_gateup_swiglu(gu[:-16], w.inter, w.hidden, x)
    with pytest.raises(ValueError):                      # x not whole rows
        tt.mxfp4_gateup_swiglu(gu, w.inter, w.hidden, x.reshape(-1)[:-8])
    with pytest.raises(ValueError):                      # bank of 3 experts holds 1
        ids = torch.zeros((2, 2), dtype=torch.int32, device=dev)
        tt.moe_mxfp4_gateup_swiglu(gu, 3, w.inter, w.hidden, x, ids)
    dn = dev_u8(tt.pack_mxfp4_matrix(*workloads.mxfp4_matrix(9, 0, w.hidden, w.inter, "down"),
                                     w.hidden, w.inter), dev)
    h = torch.zeros((2, 2, w.inter), device=dev)
    ids = torch.zeros((2, 2), dtype=torch.int32, device=dev)
    wt = torch.ones((2, 2), device=dev)
    with pytest.raises(ValueError):                      # h of the wrong shape
        tt.moe_mxfp4_down_combine(dn, 1, w.hidden, w.inter, h[:, :1].contiguous(), ids, wt)
    with pytest.raises(ValueError):                      # y too short
        tt.moe_mxfp4_down_combine(dn, 1, w.hidden, w.inter, h, ids, wt,
                                  out=torch.empty((1, w.hidden), device=dev))
    q4 = dev_u8(tt.pack_int4(*tt.quantize_int4_affine(workloads.int4_source(9, 0, 40, 256)),
                             40, 256), dev)
    with pytest.raises(ValueError):
        tt.int4_gemv(q4, 40, 256, x, out=torch.empty((2, 39), device=dev))
    # the valid calls still run
    tt.mxfp4_gateup_swiglu(gu, w.inter, w.hidden, x)
    tt.int4_gemv(q4, 40, 256, x)
    torch.cuda.synchronize()
