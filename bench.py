"""Benchmark: decode attention over a q8_0 KV cache on one MI355X.

Default run (one JSON line on stdout):
  * value: device-resident decode-attention K/V throughput (GB/s) on the
    4096-row, 40/8-head, head_dim-128 workload.  One step = attention over 64
    distinct layer caches of that shape (570 MB, more than the 256 MB
    Infinity Cache, so the data comes from HBM), launched from a captured HIP
    graph so host launch overhead stays out of the timed region.  Inputs are
    resident in HBM before timing starts.
  * roofline: the decode kernel's algorithmic bytes per launch (visible K+V
    rows + q + out) over its average launch duration (HIP events on the
    launch stream), against 8 TB/s.
  * cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
    sample of the same workload.
  * pipeline: per-token time of the host-resident 64-layer stack at 16384
    rows, ordered (depth 0) vs pipelined (depth 1, 128 MiB ring), with the
    measured pinned host-to-device link peak.
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention K/V GB/s (% of HBM/host-link peak); ms/token ordered vs pipelined"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n_rows, n_head_kv, head_dim, n_head_q, n_seq=1):
    """Visible K+V rows (each read once per KV head) plus q and out."""
    row = n_head_kv * head_dim // 32 * 34
    return n_seq * (2 * n_rows * row + 2 * n_head_q * head_dim * 4)


# ---------------------------------------------------------------- device-resident

def device_resident(args, torch, kvd, inputs):
    c = inputs.config(1)
    L = args.layers
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(c.seed)
    ks, vs, qs, outs = [], [], [], []
    for layer in range(L):
        r = c.layer_rng(layer)
        ks.append(torch.from_numpy(inputs.random_kv_rows(r, c.n_ctx, c.n_head_kv, c.head_dim)).to(dev))
        vs.append(torch.from_numpy(inputs.random_kv_rows(r, c.n_ctx, c.n_head_kv, c.head_dim)).to(dev))
        qs.append(torch.from_numpy(inputs.random_q(r, 1, c.n_head_q, c.head_dim)).to(dev))
        outs.append(torch.empty_like(qs[-1]))
    del rng
    stream = torch.cuda.Stream(device=dev)
    ws = kvd.Workspace()
    # eager warm-up (also allocates the workspace outside capture)
    with torch.cuda.stream(stream):
        for l in range(L):
            kvd.attend_decode(qs[l], outs[l], [[(ks[l], vs[l], 0)]], c.n_head_kv, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for l in range(L):
            kvd.attend_decode(qs[l], outs[l], [[(ks[l], vs[l], 0)]], c.n_head_kv, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_step = ms / args.steps
    launches = args.steps * L
    us_launch = ms * 1e3 / launches
    per_launch = algorithmic_bytes(c.n_ctx, c.n_head_kv, c.head_dim, c.n_head_q)
    gbs = per_launch / (us_launch * 1e-6) / 1e9
    # the replayed graph recomputes every layer's output; check one against eager
    ref = torch.empty_like(outs[0])
    with torch.cuda.stream(stream):
        kvd.attend_decode(qs[0], ref, [[(ks[0], vs[0], 0)]], c.n_head_kv, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    if not torch.equal(ref, outs[0]):
        raise RuntimeError("graph replay output differs from the eager call")
    curve = {}
    if args.curve:
        for n in (16384, 32768, 131072):
            curve[str(n)] = device_curve_point(torch, kvd, inputs, n, stream, ws)
        for w in (0, 4096):
            curve["batched_16seq_w%d" % w] = batched_device_point(torch, kvd, inputs, stream, ws, w)
    return {
        "ms_per_step": ms_step, "value": gbs, "us_per_launch": us_launch, "bytes_per_launch": per_launch,
        "layers_per_step": L, "curve": curve,
        "ws": ws, "q": qs[0], "k": ks[0], "v": vs[0],
    }


def batched_device_point(torch, kvd, inputs, stream, ws, window):
    """One call over the 16-sequence batch (lognormal lengths, two segments per
    sequence: older and newer halves), every row device-resident: GB/s of the
    visible K/V rows.  8 distinct layer caches cycled."""
    from decode_attention_offloaded_amd.batched import cfg4_lengths
    c = inputs.config(4)
    dev = torch.device("cuda:0")
    lens = cfg4_lengths(c)
    reps = 8
    layers = []
    for i in range(reps):
        r = np.random.default_rng([c.seed, 2000 + i])
        segs = []
        for n in lens:
            n = int(n)
            k = torch.from_numpy(inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)).to(dev)
            v = torch.from_numpy(inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)).to(dev)
            h = n // 2
            segs.append([(k[:h], v[:h], 0), (k[h:], v[h:], h)])
        q = torch.from_numpy(inputs.random_q(r, len(lens), c.n_head_q, c.head_dim)).to(dev)
        layers.append((q, segs))
    out = torch.empty_like(layers[0][0])
    with torch.cuda.stream(stream):
        for q, segs in layers:
            kvd.attend_decode(q, out, segs, c.n_head_kv, window=window, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for q, segs in layers:
            kvd.attend_decode(q, out, segs, c.n_head_kv, window=window, workspace=ws, stream=stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nrep = 5
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(nrep):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (nrep * reps)
    vis = sum(min(int(n), window) if window else int(n) for n in lens)
    b = 2 * vis * c.row_bytes + 2 * len(lens) * c.n_head_q * c.head_dim * 4
    del layers
    torch.cuda.empty_cache()
    return {"us_per_launch": round(us, 3), "visible_rows": vis, "GBps": round(b / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def device_curve_point(torch, kvd, inputs, n, stream, ws):
    """GB/s of one launch over n rows, 8 distinct layers cycled (>= 285 MB apart)."""
    c = inputs.config(1)
    dev = torch.device("cuda:0")
    reps = max(2, min(16, int(2.5e9 // (2 * n * c.row_bytes))))
    ks, vs = [], []
    for i in range(reps):
        r = np.random.default_rng([c.seed, 1000 + i, n])
        ks.append(torch.from_numpy(inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)).to(dev))
        vs.append(torch.from_numpy(inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)).to(dev))
    # a query per layer, as in a decode step (a query reused across calls stays cached)
    qs = [torch.from_numpy(inputs.random_q(np.random.default_rng([n, i]), 1, c.n_head_q, c.head_dim)).to(dev)
          for i in range(reps)]
    out = torch.empty_like(qs[0])
    with torch.cuda.stream(stream):
        for i in range(reps):
            kvd.attend_decode(qs[i], out, [[(ks[i], vs[i], 0)]], c.n_head_kv, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            kvd.attend_decode(qs[i], out, [[(ks[i], vs[i], 0)]], c.n_head_kv, workspace=ws, stream=stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nrep = 5
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(nrep):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (nrep * reps)
    b = algorithmic_bytes(n, c.n_head_kv, c.head_dim, c.n_head_q)
    del ks, vs
    torch.cuda.empty_cache()
    return {"us_per_launch": round(us, 3), "GBps": round(b / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- host link + pipeline

def link_peak(torch):
    """Pinned host -> device copy bandwidth (GB/s): one copy on one stream at
    1 MiB ... 1 GiB, and two equal copies on two streams at once (the ring's
    configuration: K and V on their own DMA engines); median of 10 timed runs
    (5 at 1 GiB) after one untimed.  The peak is the best plateau."""
    dev = torch.device("cuda:0")
    res = {}
    s0, s1 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)

    def run(n, streams):
        hs = [torch.empty(n, dtype=torch.uint8, pin_memory=True) for _ in streams]
        ds = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in streams]
        times = []
        for _ in range(11 if n <= (256 << 20) else 6):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s, h, d in zip(streams, hs, ds):
                with torch.cuda.stream(s):
                    d.copy_(h, non_blocking=True)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        t = float(np.median(times[1:]))
        return round(n * len(streams) / t / 1e9, 2)

    for mib in (1, 16, 64, 256, 1024):
        res["1x%dMiB" % mib] = run(mib << 20, [s0])
    for mib in (16, 64, 256):
        res["2x%dMiB" % mib] = run(mib << 20, [s0, s1])
    return res


def link_environment(torch):
    """Where the link figures come from: the GPU's PCI address and NUMA node,
    the NUMA nodes of the CPUs this process may run on (pinned buffers are
    allocated from them), and whether HIP's host-to-device copies use the SDMA
    engines (HSA_ENABLE_SDMA unset or not 0).  Fields that the system does not
    expose are None."""
    info = {"gpu_pci": None, "gpu_numa_node": None, "process_numa_nodes": None}
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = "%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
        info["gpu_pci"] = bdf
        with open("/sys/bus/pci/devices/%s/numa_node" % bdf) as f:
            info["gpu_numa_node"] = int(f.read().strip())
    except (OSError, ValueError, AttributeError):
        pass
    try:
        cpus = os.sched_getaffinity(0)
        nodes = set()
        for path in glob.glob("/sys/devices/system/node/node*/cpulist"):
            node = int(path.split("/node")[-1].split("/")[0])
            with open(path) as f:
                for part in f.read().strip().split(","):
                    if not part:
                        continue
                    lo, _, hi = part.partition("-")
                    if cpus & set(range(int(lo), int(hi or lo) + 1)):
                        nodes.add(node)
        info["process_numa_nodes"] = sorted(nodes) or None
    except (OSError, ValueError):
        pass
    sdma = os.environ.get("HSA_ENABLE_SDMA")
    info["HSA_ENABLE_SDMA"] = sdma
    info["sdma_copies"] = sdma is None or sdma != "0"
    return info


def pipeline(args, torch, kvd, inputs, link):
    """Host-resident 64-layer stack at 16384 rows: ordered (depth 0) vs pipelined
    (depth 1, 128 MiB ring), against the pinned H2D link peak measured here."""
    from decode_attention_offloaded_amd import stack
    peak = max(link.values())
    log("pinned H2D link: %s GB/s" % link)
    c = inputs.config(2)
    res = stack.run_host_resident(torch, kvd, inputs, c, n_layers=args.pipe_layers, depths=(0, 1, "1x"),
                                  budget_bytes=128 << 20, tokens=args.pipe_tokens, warmup=3, log=log)
    res["link_GBps_by_MiB"] = link
    res["link_peak_GBps"] = peak
    res["link_environment"] = link_environment(torch)
    for arm in res["arms"].values():
        arm["frac_link"] = round(arm["staged_GBps"] / peak, 4)
    return res


def batched(args, torch, kvd, inputs, link):
    """16 sequences of lognormal lengths, 64 layers (odd layers: 4096-row window),
    older half of every sequence staged from pinned host memory through a
    depth-1 ring (1 GiB budget), newer half device-resident: ordered vs
    pipelined per-token time."""
    from decode_attention_offloaded_amd import batched as bt
    c = inputs.config(4)
    res = bt.run_batched(torch, kvd, inputs, c, n_layers=args.batched_layers, depths=(0, 1),
                         budget_bytes=1 << 30, tokens=args.batched_tokens, warmup=2, log=log,
                         distinct_layers=4)
    peak = max(link.values())
    res["link_peak_GBps"] = peak
    for arm in res["arms"].values():
        arm["frac_link"] = round(arm["staged_GBps"] / peak, 4)
    log("batched: %s" % {k: (v["ms_per_token"], v["staged_GBps"]) for k, v in res["arms"].items()})
    return res


def tiled(args, torch, kvd, inputs, link):
    """131072 rows x 64 layers host-resident at a 128 MiB budget, where a
    whole-layer ring declines: each layer streamed in tiles through a depth-1
    ring instead (ordered tiles vs pipelined tiles)."""
    from decode_attention_offloaded_amd import tiled as tl
    c = inputs.config(3)
    res = tl.run_tiled(torch, kvd, inputs, c, n_layers=args.tiled_layers, depths=(0, 1), budget_bytes=128 << 20,
                       tokens=args.tiled_tokens, warmup=2, log=log, distinct_layers=4)
    res.pop("outs", None)
    peak = max(link.values())
    res["link_peak_GBps"] = peak
    for arm in res["arms"].values():
        arm["frac_link"] = round(arm["staged_GBps"] / peak, 4)
    log("tiled (%d rows per tile, %d tiles per layer): %s" % (res["tile_rows"], res["tiles_per_layer"], {
        k: (v["ms_per_token"], v["staged_GBps"]) for k, v in res["arms"].items()}))
    return res


def layer_compute_ms(torch, kvd, inputs, n_rows, reps=10):
    """Per-layer compute of the host-resident stack: the bf16 GEMV stand-in plus
    attention over n_rows device-resident rows (the planner's compute_ms)."""
    c = inputs.config(3)
    dev = torch.device("cuda:0")
    m, n = c.extra.get("gemv", (5120, 27648))
    w = torch.randn(m, n, dtype=torch.bfloat16, device=dev) * 0.02
    x = torch.randn(1, m, dtype=torch.bfloat16, device=dev)
    y = torch.empty(1, n, dtype=torch.bfloat16, device=dev)
    r = np.random.default_rng([c.seed, 555])
    k = torch.from_numpy(inputs.random_kv_rows(r, n_rows, c.n_head_kv, c.head_dim)).to(dev)
    v = torch.from_numpy(inputs.random_kv_rows(r, n_rows, c.n_head_kv, c.head_dim)).to(dev)
    q = torch.from_numpy(inputs.random_q(r, 1, c.n_head_q, c.head_dim)).to(dev)
    out = torch.empty_like(q)
    for _ in range(2):
        torch.matmul(x, w, out=y)
        kvd.attend_decode(q, out, [[(k, v, 0)]], c.n_head_kv)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(x, w, out=y)
        kvd.attend_decode(q, out, [[(k, v, 0)]], c.n_head_kv)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def residency(args, torch, kvd, inputs, link):
    """131072 rows x 64 layers: what a device-memory budget buys -- the
    residency planner's choice against the other option, measured."""
    from decode_attention_offloaded_amd import stack
    c = inputs.config(3)
    L, n = args.residency_layers, c.n_ctx
    lb = 2 * n * c.row_bytes
    peak = max(link.values())
    cms = layer_compute_ms(torch, kvd, inputs, n)
    arms, plans = [], {}
    for gib in (1, 4):
        budget = gib << 30
        plan = kvd.plan_residency(L, lb, budget, 1, peak, cms)
        ring_k = max(0, min(L - 1, (budget - 3 * lb) // lb)) if budget >= 3 * lb else None
        ord_k = min(L, budget // lb)
        plans[str(gib)] = plan
        if ring_k is not None:
            arms.append(("%dGiB_ring+%d" % (gib, ring_k), 1, budget, ring_k))
        arms.append(("%dGiB_ordered+%d" % (gib, ord_k), 0, 0, ord_k))
    res = stack.run_residency(torch, kvd, inputs, c, arms, n_layers=L, tokens=args.residency_tokens, warmup=2,
                              log=log, distinct_layers=4)
    res["compute_ms_per_layer"] = round(cms, 4)
    res["link_peak_GBps"] = peak
    res["plans"] = plans
    for gib, plan in plans.items():
        pick = "%sGiB_%s+%d" % (gib, "ring" if plan["use_ring"] else "ordered", plan["n_resident"])
        plan["picked_arm"] = pick
        plan["picked_is_fastest"] = bool(min((v["ms_per_token"], k) for k, v in res["arms"].items()
                                             if k.startswith(gib + "GiB"))[1] == pick)
    log("residency: %s; plans %s" % ({k: v["ms_per_token"] for k, v in res["arms"].items()},
                                     {k: v["picked_arm"] for k, v in plans.items()}))
    return res


def asymmetric(args, torch, kvd, inputs, link):
    """q8_0 K with q4_0 V: the 16384-row, 64-layer host-resident stack (ordered vs
    pipelined, 128 MiB ring), and the device-resident 4096-row call."""
    from decode_attention_offloaded_amd import stack
    c = inputs.config(2)
    res = stack.run_host_resident(torch, kvd, inputs, c, n_layers=args.pipe_layers, depths=(0, 1),
                                  budget_bytes=128 << 20, tokens=args.pipe_tokens, warmup=3, log=log, v_type=1)
    peak = max(link.values())
    res["link_peak_GBps"] = peak
    for arm in res["arms"].values():
        arm["frac_link"] = round(arm["staged_GBps"] / peak, 4)
    # device-resident 4096 rows, 64 distinct layers per graph, a query per layer
    c1 = inputs.config(1)
    dev = torch.device("cuda:0")
    L, n = 64, c1.n_ctx
    vrb = inputs.row_bytes_q4_0(c1.n_head_kv, c1.head_dim)
    ks, vs, qs = [], [], []
    for l in range(L):
        r = np.random.default_rng([c1.seed, 900 + l])
        ks.append(torch.from_numpy(inputs.random_kv_rows(r, n, c1.n_head_kv, c1.head_dim)).to(dev))
        vs.append(torch.from_numpy(inputs.random_kv_rows_q4_0(r, n, c1.n_head_kv, c1.head_dim)).to(dev))
        qs.append(torch.from_numpy(inputs.random_q(r, 1, c1.n_head_q, c1.head_dim)).to(dev))
    out = torch.empty_like(qs[0])
    stream = torch.cuda.Stream(device=dev)
    ws = kvd.Workspace()
    def call(l):
        kvd.attend_decode(qs[l], out, [[(ks[l], vs[l], 0)]], c1.n_head_kv, workspace=ws, stream=stream,
                          v_type=kvd.TYPE_Q4_0)
    with torch.cuda.stream(stream):
        for l in range(L):
            call(l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for l in range(L):
            call(l)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * L)
    b = n * (c1.row_bytes + vrb) + 2 * c1.n_head_q * c1.head_dim * 4
    res["device_4096"] = {"us_per_launch": round(us, 3), "bytes_per_launch": b,
                          "GBps": round(b / (us * 1e-6) / 1e9, 1), "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log("asymmetric q8_0 K / q4_0 V: stack %s; 4096-row call %.2f us" % (
        {k: (v["ms_per_token"], v["staged_GBps"]) for k, v in res["arms"].items()}, us))
    return res


def head_split(args, torch, kvd, inputs, link):
    """131072 rows x 64 layers, about 6.8 GB of device memory spent on residency
    two ways: 3 of 8 KV heads resident in every layer (the rest staged through
    a depth-1 ring) against 24 of 64 layers resident (the rest through a
    depth-1 ring).  Both stage 5/8 of the bytes."""
    from decode_attention_offloaded_amd import headsplit, stack
    c = inputs.config(3)
    L = args.residency_layers
    peak = max(link.values())
    hs = headsplit.run_headsplit(torch, kvd, inputs, c, 3, n_layers=L, depths=(0, 1), budget_bytes=1 << 30,
                                 tokens=args.residency_tokens, warmup=2, log=log, distinct_layers=4)
    k_layers = L * 3 // 8
    ls = stack.run_residency(torch, kvd, inputs, c, [("ring+%d" % k_layers, 1, 1 << 30, k_layers),
                                                     ("ordered+%d" % k_layers, 0, 0, k_layers)],
                             n_layers=L, tokens=args.residency_tokens, warmup=2, log=log, distinct_layers=4)
    for arm in hs["arms"].values():
        arm["frac_link"] = round(arm["staged_GBps"] / peak, 4)
    log("head split 3/8: %s; layer split %d/%d: %s" % (
        {k: v["ms_per_token"] for k, v in hs["arms"].items()}, k_layers, L,
        {k: v["ms_per_token"] for k, v in ls["arms"].items()}))
    return {"head_split": hs, "layer_split": ls, "link_peak_GBps": peak}


def long_context(args, torch, kvd, inputs):
    """131072 rows x 64 layers host-resident: depth 0/1/2 x budget 128 MiB / 1 GiB."""
    from decode_attention_offloaded_amd import stack
    c = inputs.config(3)
    out = {}
    for budget_mib in (128, 1024):
        r = stack.run_host_resident(torch, kvd, inputs, c, n_layers=args.pipe_layers, depths=(0, 1, 2),
                                    budget_bytes=budget_mib << 20, tokens=args.long_tokens, warmup=2, log=log,
                                    distinct_layers=4)
        out[str(budget_mib)] = r
        log("long context, budget %d MiB: %s" % (budget_mib, {k: (v["ms_per_token"], v["declined"])
                                                              for k, v in r["arms"].items()}))
    return out


def hbm_stream_ceiling(torch, gib=4, reps=7):
    """GB/s of plain streaming on this device: torch's elementwise negation of
    a `gib` GiB float32 tensor into another (reads and writes every byte once;
    of torch's kernels it streams fastest here: its reductions reach ~4 TB/s),
    median of `reps` runs.  A measured ceiling beside the 8 TB/s spec."""
    n = gib << 30
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(x, out=y)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del x, y
    torch.cuda.empty_cache()
    ms = sorted(times)[len(times) // 2]
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": "torch.neg, %d GiB float32 read + %d GiB written, median of %d" % (gib, gib, reps)}


def stream_same_bytes(torch, nbytes, reps=20):
    """The rate a single streaming launch of one decode call's size reaches
    here: torch's elementwise negation reading nbytes / 2 and writing nbytes / 2,
    graph-replayed over distinct buffers (at least 2.5 GB in all, as the decode
    calls cycle distinct layers), so launch and first-byte latency weigh as
    they do for a call.  Returns {"bytes", "us", "GBps", "frac_of_peak"}."""
    n = nbytes // 8
    count = max(4, min(64, int(2.5e9 // nbytes)))
    xs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(count)]
    ys = [torch.empty_like(x) for x in xs]
    s = torch.cuda.Stream(device=torch.device("cuda:0"))
    with torch.cuda.stream(s):
        for x, y in zip(xs, ys):
            torch.neg(x, out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for x, y in zip(xs, ys):
            torch.neg(x, out=y)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * count)
    del xs, ys, g
    torch.cuda.empty_cache()
    moved = 8 * n
    gbs = moved / (us * 1e-6) / 1e9
    return {"bytes": moved, "us": round(us, 3), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def calibration_copy(torch, mib=256):
    """A plain device-to-device copy of known size: the reference that hardware
    fetch/write counters are scaled by when the traffic of the decode kernel is
    measured with rocprofv3 --pmc (same process, same run)."""
    n = mib << 20
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    b = torch.empty_like(a)
    torch.neg(a, out=b)  # one elementwise kernel: reads n bytes, writes n bytes
    torch.cuda.synchronize()
    return n


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(target_s=15.0):
    import oracle
    from decode_attention_offloaded_amd import inputs
    c = inputs.config(1)
    cores = len(os.sched_getaffinity(0))
    r = c.layer_rng(0)
    k = inputs.random_kv_rows(r, c.n_ctx, c.n_head_kv, c.head_dim)
    v = inputs.random_kv_rows(r, c.n_ctx, c.n_head_kv, c.head_dim)
    q = inputs.random_q(r, 1, c.n_head_q, c.head_dim)
    t0 = time.perf_counter()
    oracle.attend(q, [[(k, v, 0)]], c.n_head_kv, c.head_dim, threads=cores)
    one = time.perf_counter() - t0
    reps = max(1, int(target_s / max(one, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.attend(q, [[(k, v, 0)]], c.n_head_kv, c.head_dim, threads=cores)
    dt = time.perf_counter() - t0
    b = algorithmic_bytes(c.n_ctx, c.n_head_kv, c.head_dim, c.n_head_q)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(b * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d calls of the 4096-row, 40/8-head, head_dim-128 layer (fp64 oracle, OpenMP over "
                      "query heads), %.1f s; %s" % (reps, dt, cpu),
            "ms_per_layer": round(dt / reps * 1e3, 2)}


# sources that decide the decode kernels' HBM traffic: the kernels and the split plan
TRAFFIC_SOURCES = ("kvd_attend.hip", "kvd_plan.cpp", "kvd_plan.h")


def traffic_source_sha():
    """sha256 over the code of TRAFFIC_SOURCES, in that order, with comments
    and whitespace removed (an edit of a comment does not change the kernels)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_offloaded_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def cpu_baseline_extra(target_s=10.0):
    """The oracle on more of the workloads (opt-in, --cpu-extra): the 4096-row
    layer on one core; one layer at 16384 and at 131072 rows and the
    16-sequence batch (full and 4096-row window) on every core."""
    import oracle
    from decode_attention_offloaded_amd import inputs
    from decode_attention_offloaded_amd.batched import cfg4_lengths
    cores = len(os.sched_getaffinity(0))
    res = {}

    def timed(name, q, segs, hkv, d, threads, window, b):
        t0 = time.perf_counter()
        oracle.attend(q, segs, hkv, d, threads=threads, window=window)
        one = time.perf_counter() - t0
        reps = max(1, int(target_s / max(one, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.attend(q, segs, hkv, d, threads=threads, window=window)
        dt = (time.perf_counter() - t0) / reps
        res[name] = {"ms_per_layer": round(dt * 1e3, 2), "GBps": round(b / dt / 1e9, 4), "threads": threads,
                     "calls": reps}

    for cfg, n, threads in ((1, 4096, 1), (2, 16384, cores), (3, 131072, cores)):
        c = inputs.config(cfg)
        r = c.layer_rng(0)
        k = inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)
        v = inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)
        q = inputs.random_q(r, 1, c.n_head_q, c.head_dim)
        timed("%d rows, %d thread%s" % (n, threads, "s" if threads > 1 else ""), q, [[(k, v, 0)]], c.n_head_kv,
              c.head_dim, threads, 0, algorithmic_bytes(n, c.n_head_kv, c.head_dim, c.n_head_q))
    c = inputs.config(4)
    r = c.layer_rng(0)
    lens = [int(x) for x in cfg4_lengths(c)]
    segs, nb_full, nb_win = [], 0, 0
    for n in lens:
        k = inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)
        v = inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)
        h = n // 2
        segs.append([(k[:h], v[:h], 0), (k[h:], v[h:], h)])
        nb_full += 2 * n * c.row_bytes
        nb_win += 2 * min(n, 4096) * c.row_bytes
    q = inputs.random_q(r, len(lens), c.n_head_q, c.head_dim)
    qb = 2 * len(lens) * c.n_head_q * c.head_dim * 4
    timed("16 sequences, full attention, %d threads" % cores, q, segs, c.n_head_kv, c.head_dim, cores, 0,
          nb_full + qb)
    timed("16 sequences, 4096-row window, %d threads" % cores, q, segs, c.n_head_kv, c.head_dim, cores, 4096,
          nb_win + qb)
    return {"cores": cores, "kind": "oracle", "workloads": res}


def measured_traffic():
    """HBM bytes per call from the committed counter summary, or None when the
    kernel or plan source has changed since the counters were taken."""
    prof = os.path.join(ROOT, "profiles", "decode_attention_4096rows_hbm_traffic.md")
    try:
        sha = traffic_source_sha()
        fields = {}
        for line in open(prof):
            if ":" in line and line.startswith("    "):
                k, v = line.strip().split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("source_sha256") == sha:
            return int(fields["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--curve", type=int, default=1)
    ap.add_argument("--pipeline", type=int, default=1)
    ap.add_argument("--pipe-layers", type=int, default=64)
    ap.add_argument("--pipe-tokens", type=int, default=20)
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--batched", type=int, default=1, help="run the 16-sequence mixed-residency stack")
    ap.add_argument("--batched-layers", type=int, default=64)
    ap.add_argument("--batched-tokens", type=int, default=4)
    ap.add_argument("--tiled", type=int, default=1, help="run 131072 rows at 128 MiB in ring-streamed tiles")
    ap.add_argument("--tiled-layers", type=int, default=64)
    ap.add_argument("--tiled-tokens", type=int, default=5)
    ap.add_argument("--residency", type=int, default=1, help="run the 131072-row residency-planner arms")
    ap.add_argument("--residency-layers", type=int, default=64)
    ap.add_argument("--residency-tokens", type=int, default=5)
    ap.add_argument("--asym", type=int, default=1, help="run the q8_0 K / q4_0 V legs")
    ap.add_argument("--headsplit", type=int, default=1, help="run the per-head residency split leg")
    ap.add_argument("--long", type=int, default=0, help="also run the 131072-row depth/budget sweep")
    ap.add_argument("--long-tokens", type=int, default=5)
    ap.add_argument("--cpu-extra", type=int, default=0,
                    help="also time the oracle single-threaded and on the 16384/131072-row and batched layers")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(one process drives one GPU; --gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    from decode_attention_offloaded_amd import inputs, kvd
    kvd.lib()
    log("device:", torch.cuda.get_device_name(0), kvd.version())
    calib = calibration_copy(torch)
    d = device_resident(args, torch, kvd, inputs)
    log("device-resident: %.1f GB/s, %.3f us/launch" % (d["value"], d["us_per_launch"]))
    out = {
        "metric": METRIC,
        "value": round(d["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode attention, device-resident q8_0 KV: 1 sequence x 4096 rows, 40 query / "
                               "8 KV heads, head_dim 128; one step = 64 distinct layer caches",
                   "n_ctx": 4096, "n_head_q": 40, "n_head_kv": 8, "head_dim": 128,
                   "layers_per_step": d["layers_per_step"], "kv": "q8_0 (34-byte blocks)"},
        "roofline": {"bound": "hbm", "achieved": round(d["value"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(d["value"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "decode_kernel<128,5,0,1> + combine_kernel<128> (one call)",
                     "bytes_per_launch": d["bytes_per_launch"], "us_per_launch": round(d["us_per_launch"], 3)},
        "device_curve": d["curve"],
        "hbm_stream_ceiling": hbm_stream_ceiling(torch),
        "calibration_copy_bytes": calib,
    }
    if args.curve:
        # what one streaming launch moving a call's algorithmic bytes reaches
        c1 = inputs.config(1)
        same = {}
        for n in (4096, 16384, 32768, 131072):
            same[str(n)] = stream_same_bytes(torch, algorithmic_bytes(n, c1.n_head_kv, c1.head_dim, c1.n_head_q))
        out["hbm_stream_ceiling"]["same_bytes_as_call"] = same
    log("streaming ceiling: %s" % out["hbm_stream_ceiling"])
    link = (link_peak(torch) if (args.pipeline or args.batched or args.tiled or args.residency or args.asym
                                 or args.headsplit) else None)
    if args.pipeline:
        out["pipeline"] = pipeline(args, torch, kvd, inputs, link)
    if args.batched:
        out["batched"] = batched(args, torch, kvd, inputs, link)
    if args.tiled:
        out["tiled"] = tiled(args, torch, kvd, inputs, link)
    if args.residency:
        out["residency"] = residency(args, torch, kvd, inputs, link)
    if args.asym:
        out["asymmetric"] = asymmetric(args, torch, kvd, inputs, link)
    if args.headsplit:
        out["head_split"] = head_split(args, torch, kvd, inputs, link)
    if args.long:
        out["long_context"] = long_context(args, torch, kvd, inputs)
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    if args.cpu_extra:
        out["cpu_baseline_extra"] = cpu_baseline_extra()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
