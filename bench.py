"""Benchmark of the weight-only MXFP4 / INT4 decode projections on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline): the SmolLM3-3B-shaped decode MLP gate/up,
hidden 2048, intermediate 11008, batch 1, MXFP4 gate and up with row
postscales, fused SwiGLU.  One step is one token through all 24 layers' gate/up
projections (24 calls, each on a different layer's weights, so the 577 MB
working set defeats the 256 MB Infinity Cache).  Inputs are synthetic (seeded,
workloads.py) and resident in HBM before timing starts.

Prints one JSON line: value = effective HBM GB/s over the algorithmic bytes
(each packed weight byte, E8M0 scale, postscale, activation and output once),
with us_per_call, the roofline of the kernel, the read ceiling (a plain
16-byte-load read of the same number of bytes from the same rotating buffers,
tt_stream_read) and the CPU oracle timed on the host (a reported baseline, not
a target).  The default line also carries sub-records, each timed the same
way against 8 TB/s and against its own read ceiling: the Phi-4-shaped gate/up,
the gpt-oss-20b-shaped MoE layer (each kernel alone and the two together), the
Phi-4-shaped INT4 QKV and O projections and the batched gate/up at 8 and 32
tokens (--headline-only skips them).

Other workloads (--workload): tiny, phi4 (gate/up), phi4-int4 (QKV + O),
gptoss (routing fused into the expert gate/up, then down/combine), batched
(--batch B), fp8-down (row-scaled FP8 down projection), attention
(single-token GQA attention, --context T), phi4-layer (a whole dense decode
layer as one graph), quantize (host MXFP4 quantizer).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# --graph-only: skip the eager timing (profiler runs, so that a kernel's
# traced average covers graph-replayed dispatches only)
GRAPH_ONLY = False


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gateup_bytes(inter, hidden, batch, out_bytes=4):
    codes = 2 * inter * hidden // 2
    scales = 2 * inter * hidden // 32
    ps = 2 * inter * 4
    return codes + scales + ps + batch * hidden * 2 + batch * inter * out_bytes


def mx_matrix_bytes(n, k):
    return n * k // 2 + n * k // 32 + n * 4


def int4_bytes(n, k, batch):
    return n * k // 2 + n * (-(-k // 128)) * 4 + batch * k * 2 + batch * n * 4


def moe_bytes(w, h_bytes=2):
    """Algorithmic bytes of one routed-expert layer at batch 1: (gate/up,
    down/combine).  gate/up: topk experts' gate and up matrices, x, h;
    down: topk experts' down matrices, h, y (ids and weights are a few
    bytes and left out)."""
    gu = w.topk * 2 * mx_matrix_bytes(w.inter, w.hidden) + w.hidden * 2 + w.topk * w.inter * h_bytes
    dn = w.topk * mx_matrix_bytes(w.hidden, w.inter) + w.topk * w.inter * h_bytes + w.hidden * 4
    return gu, dn


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def setup_gateup(tt, torch, dev, w, layers, batch, distinct=None):
    """Packed gate/up weights of `layers` layers on the device; the first
    `distinct` are generated, the rest are device copies of them."""
    import workloads
    distinct = layers if distinct is None else distinct
    packs = []
    for layer in range(distinct):
        g, u = workloads.gateup(w, layer)
        packs.append(torch.from_numpy(tt.pack_mxfp4_gateup(g, u, w.inter, w.hidden)).to(dev))
    while len(packs) < layers:
        packs.append(packs[len(packs) % distinct].clone())
    xs = [torch.from_numpy(workloads.activations(w.wid, layer, batch, w.hidden).view(np.int16))
          .to(dev) for layer in range(layers)]
    return packs, xs


def profiled_traffic(kernel_sources, summary):
    """HBM bytes per launch recorded in a profiles/ summary, or None when the
    kernel's sources have changed since those counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for f in kernel_sources:
        with open(os.path.join(ROOT, "bit_weight_only_mxfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    try:
        with open(os.path.join(ROOT, "profiles", summary)) as fh:
            fields = dict(ln.split(":", 1) for ln in fh if ln.startswith(("source_sha256:",
                                                                       "traffic_bytes_per_launch:")))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


# Before every timed measurement the device reads a separate 256 MB buffer
# for SETTLE_S seconds (untimed, and not a benchmark step).  After the
# host-side setup the GPU sits idle at low clocks, and the first ~15 ms of
# work after idle ran up to 8 % slower than the steady state (Phi-4 gate/up:
# 17.3-17.4 against 16.1 us per call in the first of six back-to-back
# timings; SmolLM3: 6.02 against 5.96 us).  --settle-ms 0 turns it off.
SETTLE_S = 0.1
_settle = {}


def settle(torch):
    if SETTLE_S <= 0:
        return
    import bit_weight_only_mxfp4_amd as tt
    if "buf" not in _settle:
        _settle["buf"] = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        _settle["sink"] = torch.empty(1, dtype=torch.int32, device="cuda")
    t0 = time.time()
    while time.time() - t0 < SETTLE_S:
        for _ in range(8):
            tt.stream_read(_settle["buf"], 8, sink=_settle["sink"])
        torch.cuda.synchronize()


def time_steps(torch, step, steps, warmup):
    """`steps` back-to-back steps between two events recorded on the current
    stream (the stream every call and graph replay here is launched on),
    after the device has left its idle clocks and `warmup` untimed steps."""
    settle(torch)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3  # seconds


def capture(torch, step):
    """One step captured as a HIP graph (the decode loop's launch path)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def time_graph(torch, step, steps, warmup):
    """Seconds for `steps` replays of `step` captured as one graph."""
    return time_steps(torch, capture(torch, step).replay, steps, warmup)


def rate(nbytes, seconds_per_call):
    """GB/s and fraction of 8 TB/s for nbytes moved per call."""
    gbs = nbytes / seconds_per_call / 1e9
    return round(gbs, 2), round(gbs / PEAK_HBM_GBS, 4)


# ---- read ceiling --------------------------------------------------------------

def read_ceiling(tt, torch, bufs, nbytes, K, W, loads=4, calls=None):
    """A plain 16-byte-load read of nbytes from each of `bufs` in turn (the
    same rotating buffers the kernel streams), `calls` reads per graph (one
    per buffer by default) as the kernel's calls are captured: seconds per
    read.  A buffer shorter than nbytes (a weight pack without the call's
    activations and outputs) is read whole."""
    nbytes = min([nbytes] + [b.numel() for b in bufs])
    nbytes -= nbytes % 16
    calls = calls or len(bufs)
    sink = torch.empty(1, dtype=torch.int32, device=bufs[0].device)

    def step():
        for c in range(calls):
            tt.stream_read(bufs[c % len(bufs)], loads, sink=sink, nbytes=nbytes)

    return time_graph(torch, step, K, W) / (K * calls), nbytes


def best_read_loads(tt, torch, bufs, nbytes, K, W):
    """Loads per lane (1, 2, 4, 8) of the fastest plain read for this size;
    returns (loads, {loads: us per read})."""
    sweep = {u: read_ceiling(tt, torch, bufs, nbytes, K, W, u)[0] for u in (1, 2, 4, 8)}
    best = min(sweep, key=sweep.get)
    return best, {str(u): round(t * 1e6, 3) for u, t in sweep.items()}


def vs_ceiling(rec, kernel_s, ceiling):
    """Adds the read ceiling (seconds, bytes read) to a record: the plain
    read's time and rate, and the fraction of it the kernel reaches (ceiling
    time over kernel time; the read covers the kernel's bytes, or its whole
    weight buffer when that is shorter)."""
    ceil_s, nread = ceiling
    gbs, frac = rate(nread, ceil_s)
    rec["read_ceiling"] = dict(us=round(ceil_s * 1e6, 3), bytes=nread, gbs=gbs,
                               frac_of_peak=frac)
    rec["frac_of_ceiling"] = round(ceil_s / kernel_s, 4)
    return rec


# ---- workloads -------------------------------------------------------------------

# decoder layers of the models the workloads are shaped like: one step (one
# graph) holds one call per layer, cycling over the rotating weight copies
MODEL_LAYERS = {"phi4": 40}


def measure_gateup(tt, torch, dev, w, batch, K, W, distinct=None, loads=4, ceiling=True,
                   calls=None):
    """Dense gate/up SwiGLU over `w.layers` rotating layers, one graph per
    step of `calls` calls (default one per rotating layer) cycling over
    them.  loads = 0 sweeps the read ceiling's loads per lane on these
    buffers and keeps the fastest.  Returns (record, per-call seconds)."""
    layers = w.layers
    calls = calls or layers
    log(f"setup {w.name}: {layers} layers ({distinct or layers} generated), batch {batch}, "
        f"{calls} calls per step")
    packs, xs = setup_gateup(tt, torch, dev, w, layers, batch, distinct)
    outs = [torch.empty((batch, w.inter), dtype=torch.float32, device=dev)
            for _ in range(layers)]

    def step():
        for c in range(calls):
            i = c % layers
            tt.mxfp4_gateup_swiglu(packs[i], w.inter, w.hidden, xs[i], out=outs[i])

    eager = None if GRAPH_ONLY else time_steps(torch, step, K, W) / (K * calls)
    per_call = time_graph(torch, step, K, W) / (K * calls)
    nbytes = gateup_bytes(w.inter, w.hidden, batch)
    gbs, frac = rate(nbytes, per_call)
    rec = dict(workload=w.name, hidden=w.hidden, inter=w.inter, batch=batch,
               us_per_call=round(per_call * 1e6, 3),
               us_per_call_eager=None if eager is None else round(eager * 1e6, 3),
               bytes_per_call=nbytes, gbs=gbs, frac_of_peak=frac,
               kernel="k_gateup_mx" if batch <= 2 else "k_gateup_mfma",
               layers_rotated=layers, calls_per_step=calls)
    if ceiling:
        if not loads:
            loads, rec["read_sweep_us"] = best_read_loads(tt, torch, packs, nbytes, K, W)
        rec["read_loads_per_lane"] = loads
        vs_ceiling(rec, per_call, read_ceiling(tt, torch, packs, nbytes, K, W, loads, calls))
    return rec, per_call


def measure_moe(tt, torch, dev, K, W, loads=4):
    """The gpt-oss-20b-shaped routed-expert layer at batch 1 over 24 rotating
    layers (copies of one generated 32-expert bank, a distinct routing per
    layer): routing fused into the expert gate/up, then down + combine; each
    kernel alone and the whole layer, one graph per step."""
    import workloads
    w = workloads.GPTOSS
    layers, E = w.layers, w.n_experts
    log(f"setup {w.name}: 1 generated layer of {E} experts, {layers} device copies")
    gb = workloads.expert_bank(w, 0, "gate")
    ub = workloads.expert_bank(w, 0, "up")
    db = workloads.expert_bank(w, 0, "down")
    gs = tt.mxfp4_gateup_pack_bytes(w.inter, w.hidden)
    ds = tt.mxfp4_matrix_pack_bytes(w.hidden, w.inter)
    gu = np.empty(E * gs, np.uint8)
    dn = np.empty(E * ds, np.uint8)
    for e in range(E):
        tt.pack_mxfp4_gateup((gb[0][e], gb[1][e], gb[2][e]), (ub[0][e], ub[1][e], ub[2][e]),
                             w.inter, w.hidden, out=gu[e * gs:(e + 1) * gs])
        tt.pack_mxfp4_matrix(db[0][e], db[1][e], db[2][e], w.hidden, w.inter,
                             out=dn[e * ds:(e + 1) * ds])
    del gb, ub, db
    gu0 = torch.from_numpy(gu).to(dev)
    dn0 = torch.from_numpy(dn).to(dev)
    del gu, dn
    banks = [(gu0, dn0)] + [(gu0.clone(), dn0.clone()) for _ in range(layers - 1)]
    logits = [torch.from_numpy(workloads.router_logits(w.wid, s, 1, E).view(np.int16)).to(dev)
              for s in range(layers)]
    x = torch.from_numpy(workloads.activations(w.wid, 0, 1, w.hidden).view(np.int16)).to(dev)
    ids = [torch.empty((1, w.topk), dtype=torch.int32, device=dev) for _ in range(layers)]
    wt = [torch.empty((1, w.topk), dtype=torch.float32, device=dev) for _ in range(layers)]
    h = [torch.empty((1, w.topk, w.inter), dtype=torch.bfloat16, device=dev)
         for _ in range(layers)]
    y = torch.empty((1, w.hidden), dtype=torch.float32, device=dev)

    def gateup_step():
        for li, (g_, _) in enumerate(banks):
            tt.moe_mxfp4_route_gateup_swiglu(g_, E, w.inter, w.hidden, x, logits[li], w.topk,
                                             ids=ids[li], w=wt[li], out=h[li])

    def down_step():
        for li, (_, d_) in enumerate(banks):
            tt.moe_mxfp4_down_combine(d_, E, w.hidden, w.inter, h[li], ids[li], wt[li], out=y)

    def layer_step():
        for li, (g_, d_) in enumerate(banks):
            tt.moe_mxfp4_route_gateup_swiglu(g_, E, w.inter, w.hidden, x, logits[li], w.topk,
                                             ids=ids[li], w=wt[li], out=h[li])
            tt.moe_mxfp4_down_combine(d_, E, w.hidden, w.inter, h[li], ids[li], wt[li], out=y)

    layer_s = time_graph(torch, layer_step, K, W) / (K * layers)
    gu_s = time_graph(torch, gateup_step, K, W) / (K * layers)   # leaves ids, w, h per layer
    dn_s = time_graph(torch, down_step, K, W) / (K * layers)
    gu_b, dn_b = moe_bytes(w)
    gu_c = read_ceiling(tt, torch, [b[0] for b in banks], gu_b, K, W, loads)
    dn_c = read_ceiling(tt, torch, [b[1] for b in banks], dn_b, K, W, loads)
    both = gu_c[0] + dn_c[0]
    lay_gbs, lay_frac = rate(gu_b + dn_b, layer_s)
    rec = dict(workload=w.name, hidden=w.hidden, inter=w.inter, experts=E, topk=w.topk,
               batch=1, h_dtype="bf16", layers_rotated=layers,
               us_per_layer=round(layer_s * 1e6, 3), bytes_per_layer=gu_b + dn_b,
               gbs=lay_gbs, frac_of_peak=lay_frac,
               read_ceiling=dict(us=round(both * 1e6, 3),
                                 note="the two reads, one launch each"),
               frac_of_ceiling=round(both / layer_s, 4),
               kernels={})
    for name, kern, nb, s, c in (("gateup_routed", "k_gateup_mx (routing fused)", gu_b, gu_s,
                                  gu_c),
                                 ("down_combine", "k_down_mx", dn_b, dn_s, dn_c)):
        gbs, frac = rate(nb, s)
        rec["kernels"][name] = vs_ceiling(dict(kernel=kern, us_per_call=round(s * 1e6, 3),
                                               bytes_per_call=nb, gbs=gbs, frac_of_peak=frac),
                                          s, c)
    return rec, layer_s


def measure_int4(tt, torch, dev, K, W, loads=4):
    """The Phi-4-shaped INT4 QKV (7680 x 5120) and O (5120 x 5120)
    projections, one copy per Phi-4 layer (40, 1.4 GB: more than the 256 MB
    last-level cache holds), each projection timed alone."""
    import workloads
    w = workloads.PHI4
    (nq, kq), (no, ko) = workloads.attention_shapes(w)
    copies, distinct = MODEL_LAYERS["phi4"], 2
    log(f"setup INT4 QKV [{nq}x{kq}] and O [{no}x{ko}], {copies} copies")
    packs = {"qkv": [], "o": []}
    for layer in range(distinct):
        for name, (n, k, tid) in (("qkv", (nq, kq, workloads.T_INT4W)),
                                  ("o", (no, ko, workloads.T_INT4W + 100))):
            q, s, z = tt.quantize_int4_affine(workloads.int4_source(w.wid, layer, n, k, tid))
            packs[name].append(torch.from_numpy(tt.pack_int4(q, s, z, n, k)).to(dev))
    for name in packs:
        while len(packs[name]) < copies:
            packs[name].append(packs[name][len(packs[name]) % distinct].clone())
    x = torch.from_numpy(workloads.activations(w.wid, 0, 1, kq, workloads.T_OX)
                         .view(np.int16)).to(dev)
    calls = MODEL_LAYERS["phi4"]
    rec = {}
    for name, (n, k) in (("qkv", (nq, kq)), ("o", (no, ko))):
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        ps = packs[name]

        def step(ps=ps, n=n, k=k, y=y):
            for c in range(calls):
                tt.int4_gemv(ps[c % copies], n, k, x, out=y)

        s = time_graph(torch, step, K, W) / (K * calls)
        nb = int4_bytes(n, k, 1)
        gbs, frac = rate(nb, s)
        rec[name] = vs_ceiling(dict(shape=[n, k], group=128, kernel="k_int4_gemv",
                                    us_per_call=round(s * 1e6, 3), bytes_per_call=nb, gbs=gbs,
                                    frac_of_peak=frac, copies_rotated=copies,
                                    calls_per_step=calls),
                               s, read_ceiling(tt, torch, ps, nb, K, W, loads, calls))
    return rec


def cpu_baseline_gateup(w, seconds):
    """The oracle, untuned, single-threaded, on full layers of the same
    workload until about `seconds` of CPU work; then the OpenMP build of the
    same loops (rows split over the host threads, same bits) on the same
    layers for about a third of that."""
    import oracle
    import workloads

    def timed(parallel, budget):
        t_total, calls, nbytes, layer = 0.0, 0, 0, 0
        while t_total < budget and layer < w.layers:
            g, u = workloads.gateup(w, layer)
            x = workloads.activations(w.wid, layer, 1, w.hidden)
            t0 = time.perf_counter()
            oracle.mxfp4_gateup_swiglu(g, u, w.inter, w.hidden, x, parallel=parallel)
            t_total += time.perf_counter() - t0
            calls += 1
            nbytes += gateup_bytes(w.inter, w.hidden, 1)
            layer += 1
        return t_total, calls, nbytes

    t_total, calls, nbytes = timed(False, seconds)
    tp, cp, bp = timed(True, seconds / 3)
    nthr = oracle.threads(parallel=True)
    return dict(value=round(nbytes / t_total / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                cpu_model=cpu_model(), us_per_call=round(t_total / calls * 1e6, 1),
                sample=f"{calls} full {w.name} layer calls (batch 1), single thread, "
                       f"fp64 oracle, {t_total:.1f} s",
                parallel=dict(value=round(bp / tp / 1e9, 4), unit="GB/s", cores=nthr,
                              us_per_call=round(tp / cp * 1e6, 1),
                              sample=f"{cp} full {w.name} layer calls, the same oracle loops "
                                     f"with rows split over {nthr} OpenMP threads, "
                                     f"{tp:.1f} s"))


GATEUP_METRIC = "effective HBM GB/s of the MXFP4 gate/up SwiGLU GEMV (us/call alongside)"


def run(args):
    import torch

    import bit_weight_only_mxfp4_amd as tt
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup
    result = None

    if args.workload in ("smollm3", "tiny", "phi4", "batched"):
        w = {"smollm3": workloads.SMOLLM3, "tiny": workloads.TINY, "phi4": workloads.PHI4,
             "batched": workloads.BATCHED}[args.workload]
        batch = args.batch if args.workload == "batched" else 1
        distinct = min(w.layers, 4) if args.workload == "phi4" else None
        # the read ceiling's loads per lane: swept on the headline's buffers
        # (the fastest plain read of its bytes), then used for every ceiling
        rec, per_call = measure_gateup(tt, torch, dev, w, batch, K, W, distinct,
                                       args.read_loads, ceiling=args.workload != "tiny",
                                       calls=MODEL_LAYERS.get(args.workload))
        loads = rec.get("read_loads_per_lane", 4)
        calls = K * rec["calls_per_step"]
        result = dict(metric=GATEUP_METRIC, value=rec["gbs"], unit="GB/s",
                      us_per_call=rec["us_per_call"], us_per_call_eager=rec["us_per_call_eager"],
                      ms_per_step=round(per_call * rec["calls_per_step"] * 1e3, 4),
                      bytes_per_call=rec["bytes_per_call"],
                      config=dict(workload=w.name, hidden=w.hidden, inter=w.inter, batch=batch,
                                  layers_rotated=w.layers, calls_per_step=rec["calls_per_step"],
                                  launch="one HIP graph per step"),
                      roofline=dict(bound="hbm", kernel=rec["kernel"], achieved=rec["gbs"],
                                    peak=PEAK_HBM_GBS, unit="GB/s", frac=rec["frac_of_peak"],
                                    traffic=None,
                                    basis=f"algorithmic bytes per call / average per-call time "
                                          f"of {calls} graph-replayed calls (HIP events)"))
        if "read_ceiling" in rec:
            result["read_ceiling"] = dict(rec["read_ceiling"], kernel="k_stream_read",
                                          loads_per_lane=loads,
                                          sweep_us=rec.get("read_sweep_us"))
            result["frac_of_ceiling"] = rec["frac_of_ceiling"]
        if args.workload == "smollm3":
            result["roofline"]["traffic"] = profiled_traffic(
                ("mxfp4_gateup.hip", "device.h", "layout.h"), "gateup_smollm3_b1.md")
            if not args.headline_only:
                log("sub-records ...")
                sub = {}
                phi, _ = measure_gateup(tt, torch, dev, workloads.PHI4, 1, K, W, 4, loads,
                                        calls=MODEL_LAYERS["phi4"])
                sub["phi4_gateup"] = phi
                torch.cuda.empty_cache()
                sub["gptoss_moe_layer"], _ = measure_moe(tt, torch, dev, K, W, loads)
                torch.cuda.empty_cache()
                sub["phi4_int4"] = measure_int4(tt, torch, dev, K, W, loads)
                torch.cuda.empty_cache()
                # the batched config (SmolLM3 shapes) on the matrix-core path
                sub["batched_gateup"] = {}
                for b in (8, 32):
                    sub["batched_gateup"][f"batch{b}"], _ = measure_gateup(
                        tt, torch, dev, workloads.BATCHED, b, K, W, None, loads)
                    torch.cuda.empty_cache()
                result["subrecords"] = sub
        if not args.no_cpu_baseline and args.workload in ("smollm3", "tiny"):
            log("cpu baseline (oracle) ...")
            result["cpu_baseline"] = cpu_baseline_gateup(w, args.cpu_seconds)

    elif args.workload == "phi4-int4":
        rec = measure_int4(tt, torch, dev, K, W, args.read_loads or 4)
        q, o = rec["qkv"], rec["o"]
        per_pair = q["bytes_per_call"] + o["bytes_per_call"]
        secs = (q["us_per_call"] + o["us_per_call"]) * 1e-6
        gbs, frac = rate(per_pair, secs)
        result = dict(metric="effective HBM GB/s of the grouped affine INT4 GEMV (QKV + O)",
                      value=gbs, unit="GB/s", us_per_call=round(secs / 2 * 1e6, 3),
                      ms_per_step=round(secs * MODEL_LAYERS["phi4"] * 1e3, 4),
                      config=dict(workload="phi4-14b-int4-qkv-o", qkv=q["shape"], o=o["shape"],
                                  group=128, copies_rotated=16,
                                  calls_per_step=MODEL_LAYERS["phi4"],
                                  launch="one HIP graph per projection and step"),
                      roofline=dict(bound="hbm", kernel="k_int4_gemv", achieved=gbs,
                                    peak=PEAK_HBM_GBS, unit="GB/s", frac=frac,
                                    traffic=profiled_traffic(
                                        ("int4_gemv.hip", "device.h", "layout.h"),
                                        "int4_phi4_qkv_o.md")),
                      projections=rec)

    elif args.workload == "gptoss":
        rec, layer_s = measure_moe(tt, torch, dev, K, W, args.read_loads or 4)
        result = dict(metric="effective HBM GB/s of the routed-expert MXFP4 layer "
                             "(route + expert gate/up SwiGLU + down/combine)",
                      value=rec["gbs"], unit="GB/s", us_per_layer=rec["us_per_layer"],
                      ms_per_step=round(layer_s * rec["layers_rotated"] * 1e3, 4),
                      config=dict(workload=rec["workload"], hidden=rec["hidden"],
                                  inter=rec["inter"], experts=rec["experts"], topk=rec["topk"],
                                  batch=1, layers_rotated=rec["layers_rotated"], h_dtype="bf16",
                                  routing="a distinct seeded routing per layer, fused into "
                                          "the expert gate/up call",
                                  launch="one HIP graph per step"),
                      roofline=dict(bound="hbm", kernel="k_gateup_mx(routed)+k_down_mx",
                                    achieved=rec["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                                    frac=rec["frac_of_peak"],
                                    traffic=profiled_traffic(
                                        ("mxfp4_gateup.hip", "moe.hip", "device.h", "layout.h"),
                                        "moe_gptoss_layer.md")),
                      kernels=rec["kernels"], read_ceiling=rec["read_ceiling"],
                      frac_of_ceiling=rec["frac_of_ceiling"])

    elif args.workload == "fp8-down":
        # the dense down projection of the SmolLM3-shaped MLP as a row-scaled
        # FP8 matvec on the gate/up SwiGLU output h (fp32), batch 1
        n, k, layers = 2048, 11008, 24
        log(f"setup FP8 down [{n}x{k}], {layers} layers")
        packs = []
        for layer in range(4):
            codes, scale = workloads.fp8_matrix(1, layer, n, k)
            packs.append(torch.from_numpy(tt.pack_fp8_matrix(codes, scale, n, k)).to(dev))
        while len(packs) < layers:
            packs.append(packs[len(packs) % 4].clone())
        h = torch.from_numpy(workloads.swiglu_like(1, 0, 1, k)).to(dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)

        def step():
            for p in packs:
                tt.fp8_gemv(p, n, k, h, out=y)

        secs = time_graph(torch, step, K, W)
        calls = K * layers
        per_call = n * k + n * 4 + k * 4 + n * 4
        gbs, frac = rate(per_call, secs / calls)
        result = dict(metric="effective HBM GB/s of the row-scaled FP8 E4M3 down projection",
                      value=gbs, unit="GB/s", us_per_call=round(secs / calls * 1e6, 3),
                      ms_per_step=round(secs / K * 1e3, 4), bytes_per_call=per_call,
                      config=dict(workload="smollm3-3b-fp8-down-h2048-i11008", n=n, k=k,
                                  batch=1, x="fp32 SwiGLU output", layers_rotated=layers,
                                  launch="one HIP graph per step"),
                      roofline=dict(bound="hbm", kernel="k_fp8_gemv", achieved=gbs,
                                    peak=PEAK_HBM_GBS, unit="GB/s", frac=frac,
                                    traffic=profiled_traffic(
                                        ("fp8_gemv.hip", "device.h", "layout.h"),
                                        "fp8_down_smollm3.md")))
        vs_ceiling(result, secs / calls,
                   read_ceiling(tt, torch, packs, per_call, K, W, args.read_loads or 4))

    elif args.workload == "attention":
        # single-token GQA attention, Phi-4-shaped heads by default (40 query /
        # 10 kv x 128; --heads), a 4096-position bf16 KV cache per layer, 24
        # layers rotated
        hq, hkv, d = (int(v) for v in args.heads.split(","))
        T, layers = args.context, 24
        log(f"setup attention hq {hq} hkv {hkv} d {d} T {T}, {layers} layers")
        gen = np.random.default_rng([0, 77])
        caches = []
        for layer in range(2):
            kc = workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32))
            vc = workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32))
            caches.append((torch.from_numpy(kc.view(np.int16)).to(dev),
                           torch.from_numpy(vc.view(np.int16)).to(dev)))
        while len(caches) < layers:
            caches.append(tuple(c.clone() for c in caches[len(caches) % 2]))
        q = torch.from_numpy(workloads.bf16_bits(gen.standard_normal((hq, d)).astype(np.float32))
                             .view(np.int16)).to(dev)
        out = torch.empty((hq, d), dtype=torch.float32, device=dev)
        ws = torch.empty(tt.gqa_attention_workspace_bytes(hq, hkv, d, T), dtype=torch.uint8,
                         device=dev)
        scale = 1.0 / np.sqrt(d)

        def step():
            for kc_, vc_ in caches:
                tt.gqa_attention_decode(q, kc_, vc_, hq, hkv, d, T, scale, out=out, workspace=ws)

        secs = time_graph(torch, step, K, W)
        calls = K * layers
        per_call = 2 * hkv * T * d * 2 + hq * d * 2 + hq * d * 4
        gbs, frac = rate(per_call, secs / calls)
        result = dict(metric="effective HBM GB/s of single-token GQA attention over a bf16 KV "
                             "cache",
                      value=gbs, unit="GB/s", us_per_call=round(secs / calls * 1e6, 3),
                      ms_per_step=round(secs / K * 1e3, 4), bytes_per_call=per_call,
                      config=dict(workload=(f"phi4-14b-gqa-attention-40-10x128-T{T}"
                                            if (hq, hkv, d) == (40, 10, 128) else
                                            f"gqa-attention-{hq}-{hkv}x{d}-T{T}"), hq=hq,
                                  hkv=hkv, d=d, T=T, layers_rotated=layers,
                                  launch="one HIP graph per step (2 kernels per call)"),
                      roofline=dict(bound="hbm", kernel="k_attn_partial+k_attn_combine",
                                    achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s", frac=frac,
                                    traffic=profiled_traffic(
                                        ("attention.hip", "device.h"),
                                        "attention_phi4_t4096.md")
                                    if (T, hq, hkv, d) == (4096, 40, 10, 128) else None))

    elif args.workload == "phi4-layer":
        # one dense decode layer as one HIP graph, Phi-4 shapes: INT4 QKV ->
        # GQA attention (bf16 KV cache, --context positions) -> INT4 O ->
        # MXFP4 gate/up SwiGLU -> FP8 down; 8 layers rotated
        w = workloads.PHI4
        hq, hkv, d = w.heads
        T, layers, distinct = args.context, 8, 2
        (nq, kq), (no, ko) = workloads.attention_shapes(w)
        log(f"setup Phi-4-shaped decode layer, T {T}, {layers} layers ({distinct} generated)")
        gen = np.random.default_rng([0, 78])
        L = []
        for layer in range(distinct):
            qkv = tt.pack_int4(*tt.quantize_int4_affine(
                workloads.int4_source(w.wid, layer, nq, kq)), nq, kq)
            o4 = tt.pack_int4(*tt.quantize_int4_affine(
                workloads.int4_source(w.wid, layer, no, ko, workloads.T_INT4W + 100)), no, ko)
            gu = tt.pack_mxfp4_gateup(*workloads.gateup(w, layer), w.inter, w.hidden)
            dc, dsc = workloads.fp8_matrix(w.wid, layer, w.hidden, w.inter)
            dn = tt.pack_fp8_matrix(dc, dsc, w.hidden, w.inter)
            kc = workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32))
            vc = workloads.bf16_bits(gen.standard_normal((hkv, T, d)).astype(np.float32))
            L.append([torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
                      for a in (qkv, o4, gu, dn, kc, vc)])
        while len(L) < layers:
            L.append([t.clone() for t in L[len(L) % distinct]])
        x = torch.from_numpy(workloads.activations(w.wid, 0, 1, w.hidden).view(np.int16)).to(dev)
        ws = torch.empty(tt.gqa_attention_workspace_bytes(hq, hkv, d, T), dtype=torch.uint8,
                         device=dev)
        bf = torch.bfloat16
        yq = torch.empty((1, nq), dtype=bf, device=dev)
        att = torch.empty((hq, d), dtype=bf, device=dev)
        yo = torch.empty((1, no), dtype=bf, device=dev)
        h = torch.empty((1, w.inter), dtype=bf, device=dev)   # bf16 like every activation
        y = torch.empty((1, w.hidden), device=dev)

        def layer_calls(qkv, o4, gu, dn, kc, vc):
            tt.int4_gemv(qkv, nq, kq, x, out=yq)
            tt.gqa_attention_decode(yq[0, :hq * d], kc.view(bf), vc.view(bf), hq, hkv, d, T,
                                    d ** -0.5, out=att, workspace=ws)
            tt.int4_gemv(o4, no, ko, att.view(1, hq * d), out=yo)
            tt.mxfp4_gateup_swiglu(gu, w.inter, w.hidden, yo, out=h)
            tt.fp8_gemv(dn, w.hidden, w.inter, h, out=y)

        graphs = [capture(torch, lambda l=l: layer_calls(*l)) for l in L]

        def step():
            for g in graphs:
                g.replay()

        secs = time_steps(torch, step, K, W)
        per_layer = (int4_bytes(nq, kq, 1) - nq * 2 + 2 * hkv * T * d * 2 + hq * d * 2
                     + int4_bytes(no, ko, 1) - no * 2 + gateup_bytes(w.inter, w.hidden, 1, 2)
                     + w.hidden * w.inter + w.hidden * 4 + w.inter * 2 + w.hidden * 4)
        gbs, frac = rate(per_layer, secs / (K * layers))
        result = dict(metric="effective HBM GB/s of one dense decode layer run as one HIP graph "
                             "(INT4 QKV, GQA attention, INT4 O, MXFP4 gate/up SwiGLU, FP8 down)",
                      value=gbs, unit="GB/s",
                      us_per_layer=round(secs / (K * layers) * 1e6, 3),
                      ms_per_step=round(secs / K * 1e3, 4), bytes_per_layer=per_layer,
                      config=dict(workload=f"phi4-14b-decode-layer-T{T}", hidden=w.hidden,
                                  inter=w.inter, heads=[hq, hkv, d], T=T, layers_rotated=layers,
                                  launch="one HIP graph per layer (6 kernels)"),
                      roofline=dict(bound="hbm", kernel="layer graph", achieved=gbs,
                                    peak=PEAK_HBM_GBS, unit="GB/s", frac=frac, traffic=None))

    elif args.workload == "quantize":
        # host-side MXFP4 quantizer + postscale fit on one SmolLM3-shaped
        # layer's fp32 gate and up rows (a host function: no GPU work)
        w = workloads.SMOLLM3
        gen = np.random.default_rng([0, 99])
        wg = (0.02 * gen.standard_normal((w.inter, w.hidden))).astype(np.float32)
        wu = (0.02 * gen.standard_normal((w.inter, w.hidden))).astype(np.float32)
        tt.quantize_mxfp4(wg)
        t0 = time.perf_counter()
        for _ in range(K):
            tt.quantize_mxfp4(wg)
            tt.quantize_mxfp4(wu)
        secs = time.perf_counter() - t0
        nbytes = 2 * wg.nbytes
        gbs = nbytes * K / secs / 1e9
        result = dict(metric="host MXFP4 quantizer + row-postscale fit throughput (fp32 in)",
                      value=round(gbs, 3), unit="GB/s", ms_per_step=round(secs / K * 1e3, 3),
                      config=dict(workload="smollm3-3b-gateup-quantize", rows=2 * w.inter,
                                  k=w.hidden, threads=1),
                      roofline=None)
        if not args.no_cpu_baseline:
            import oracle
            t0 = time.perf_counter()
            oracle.mxfp4_quantize(wg)
            oracle.mxfp4_quantize(wu)
            osecs = time.perf_counter() - t0
            result["cpu_baseline"] = dict(value=round(nbytes / osecs / 1e9, 3), unit="GB/s",
                                          cores=1, kind="oracle", cpu_model=cpu_model(),
                                          sample="one layer's gate and up rows, single thread")
    else:
        raise SystemExit(f"unknown workload {args.workload}")

    scaled = "fp4-e2m1 x bf16 (as two e4m3 parts) on the scaled matrix instruction"
    dtype = {"phi4-int4": "int4 x bf16 -> fp32 accumulate",
             "phi4-layer": "int4 / fp4-e2m1 / fp8-e4m3 / bf16 x bf16 -> fp32 accumulate",
             "attention": "bf16 x bf16 -> fp32 accumulate",
             "fp8-down": "fp8-e4m3 x fp32 -> fp32 accumulate",
             "quantize": "fp32 -> fp4-e2m1 + e8m0 (host)"}.get(args.workload, scaled)
    if args.workload == "batched" and args.batch > 2:
        dtype = "fp4-e2m1 x bf16 -> fp32 accumulate"
    result.update(n_gpus=1, steps=K, warmup=W, higher_is_better=True, scaling="strong",
                  vs_baseline=None, dtype=dtype,
                  data="synthetic (seeded codes, scales, postscales, activations)",
                  settle_ms_before_each_timing=args.settle_ms)
    if "cpu_baseline" not in result:
        result["cpu_baseline"] = None
    order = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
             "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
             "roofline", "cpu_baseline"]
    out = {k: result[k] for k in order if k in result}
    out.update({k: v for k, v in result.items() if k not in out})
    print(json.dumps(out), flush=True)


def copy_probe(mib, reps):
    """A plain device-to-device copy of a known size (for normalising the
    HBM byte counters of a profiler run against a known transfer)."""
    import torch
    dev = torch.device("cuda", 0)
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(probe="copy", bytes_read=n, bytes_written=n, reps=reps)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="smollm3",
                    choices=["smollm3", "tiny", "phi4", "phi4-int4", "gptoss", "batched",
                             "fp8-down", "attention", "phi4-layer", "quantize"])
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--context", type=int, default=4096,
                    help="cached positions for --workload attention")
    ap.add_argument("--heads", default="40,10,128",
                    help="query heads, kv heads, head dim for --workload attention "
                         "(default Phi-4; gpt-oss-20b: 64,8,64)")
    ap.add_argument("--headline-only", action="store_true",
                    help="default workload: skip the sub-records")
    ap.add_argument("--read-loads", type=int, default=0, choices=[0, 1, 2, 4, 8],
                    help="loads per lane of the read ceiling (0: the fastest, swept)")
    ap.add_argument("--graph-only", action="store_true",
                    help="skip the eager timing (for profiler runs)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="plain reads of a separate 256 MB buffer before each timed "
                         "measurement, so that it starts at the device's working clocks "
                         "(0: off)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (profiler calibration)")
    args = ap.parse_args()
    global GRAPH_ONLY, SETTLE_S
    GRAPH_ONLY = args.graph_only
    SETTLE_S = args.settle_ms / 1e3
    if args.copy_probe:
        copy_probe(args.copy_probe, 4)
        return
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported: the "
              "projections are measured on one MI355X only.", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
