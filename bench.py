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
    rows, ordered (depth 0) vs pipelined (depth 1, 128 MiB ring), against the
    pinned host-to-device plateau probed the way the ring copies (two streams).
  * device_memory_table / long_context: the page's Device-memory table on this
    machine (4096 ... 65536 rows, ring size, device-memory growth, declines)
    and the 131072-row depth x budget sweep.
  * batched, tiled, residency, asymmetric, head_split: the other host-resident
    workloads.
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
    if args.rows != c.n_ctx:
        # another context length of the same geometry (profiling runs)
        import dataclasses
        c = dataclasses.replace(c, n_ctx=args.rows)
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
    plan_args, _keep = kvd.make_args(qs[0], outs[0], [[(ks[0], vs[0], 0)]], c.n_head_kv)
    split_rows, waves, n_splits = kvd.attend_plan(plan_args)
    load_mode = kvd.attend_load_mode(plan_args)
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
        "plan": {"split_rows": split_rows, "waves": waves, "splits": n_splits, "load_mode": load_mode},
        "ws": ws, "q": qs[0], "k": ks[0], "v": vs[0],
    }


def batched_device_point(torch, kvd, inputs, stream, ws, window, calls=64):
    """One call over the 16-sequence batch (lognormal lengths, two segments per
    sequence: older and newer halves), every row device-resident: GB/s of the
    visible K/V rows.  A graph of `calls` calls cycling 8 distinct layer caches."""
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
    seq = [layers[i % reps] for i in range(max(calls, reps))]
    with torch.cuda.stream(stream):
        for q, segs in seq:
            kvd.attend_decode(q, out, segs, c.n_head_kv, window=window, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for q, segs in seq:
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
    us = e0.elapsed_time(e1) * 1e3 / (nrep * len(seq))
    vis = sum(min(int(n), window) if window else int(n) for n in lens)
    b = 2 * vis * c.row_bytes + 2 * len(lens) * c.n_head_q * c.head_dim * 4
    del layers
    torch.cuda.empty_cache()
    return {"us_per_launch": round(us, 3), "visible_rows": vis, "GBps": round(b / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def device_curve_point(torch, kvd, inputs, n, stream, ws, calls=64):
    """GB/s of one call over n rows: a graph of `calls` calls (one decode step
    of 64 layers, as the headline measures it) cycling at least 2 and at most
    16 distinct layer caches, >= 2.5 GB between a layer's reuses."""
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
    idx = [i % reps for i in range(max(calls, reps))]
    with torch.cuda.stream(stream):
        for i in idx:
            kvd.attend_decode(qs[i], out, [[(ks[i], vs[i], 0)]], c.n_head_kv, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in idx:
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
    us = e0.elapsed_time(e1) * 1e3 / (nrep * len(idx))
    b = algorithmic_bytes(n, c.n_head_kv, c.head_dim, c.n_head_q)
    del ks, vs
    torch.cuda.empty_cache()
    return {"us_per_launch": round(us, 3), "GBps": round(b / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- host link + pipeline

def link_peak(kvd):
    """Pinned host-to-device copy rate as the ring copies (kvd_link_probe:
    hipHostMalloc'ed source, hipMemcpyAsync on non-blocking streams, HIP-event
    timed, median of 10 runs, 5 at 1 GiB): one stream, and the bytes split
    over two streams (the ring's two transfer streams, one DMA engine each),
    at 16 MiB ... 1 GiB.  Returns (figures, one-stream plateau, two-stream
    plateau)."""
    res = {}
    for mib in (16, 64, 256, 1024):
        for ns in (1, 2):
            res["%dx%dMiB" % (ns, mib)] = round(kvd.link_probe(mib << 20, ns, 10 if mib <= 256 else 5), 2)
    one = max(v for k, v in res.items() if k.startswith("1x"))
    two = max(v for k, v in res.items() if k.startswith("2x"))
    return res, one, two


def frac_link(res, link):
    """Staged GB/s of every arm over the two-stream plateau (the ring's
    configuration); ordered arms copy on one stream, so they are also given
    against the one-stream plateau."""
    figures, one, two = link
    res["link_GBps_by_size"] = figures
    res["link_plateau_1stream_GBps"] = one
    res["link_plateau_2stream_GBps"] = two
    for arm in res["arms"].values():
        gbs = arm.get("staged_GBps")
        if gbs is None:
            continue
        arm["frac_link"] = round(gbs / two, 4)
        if arm.get("depth") == 0:
            arm["frac_link_1stream"] = round(gbs / one, 4)
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
    log("pinned H2D link (GB/s): %s" % (link[0],))
    c = inputs.config(2)
    res = stack.run_host_resident(torch, kvd, inputs, c, n_layers=args.pipe_layers, depths=(0, 1, "1x"),
                                  budget_bytes=128 << 20, tokens=args.pipe_tokens, warmup=3, log=log)
    res["link_environment"] = link_environment(torch)
    return frac_link(res, link)


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
    frac_link(res, link)
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
    frac_link(res, link)
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
    peak = link[2]
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
    res["link_plateau_2stream_GBps"] = peak
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
    frac_link(res, link)
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
    hs = headsplit.run_headsplit(torch, kvd, inputs, c, 3, n_layers=L, depths=(0, 1), budget_bytes=1 << 30,
                                 tokens=args.residency_tokens, warmup=2, log=log, distinct_layers=4)
    k_layers = L * 3 // 8
    ls = stack.run_residency(torch, kvd, inputs, c, [("ring+%d" % k_layers, 1, 1 << 30, k_layers),
                                                     ("ordered+%d" % k_layers, 0, 0, k_layers)],
                             n_layers=L, tokens=args.residency_tokens, warmup=2, log=log, distinct_layers=4)
    frac_link(hs, link)
    log("head split 3/8: %s; layer split %d/%d: %s" % (
        {k: v["ms_per_token"] for k, v in hs["arms"].items()}, k_layers, L,
        {k: v["ms_per_token"] for k, v in ls["arms"].items()}))
    return {"head_split": hs, "layer_split": ls}


def golden_ring_table():
    """The [R4] Device-memory table as kept in tests/golden/ring_table.txt:
    {context: (peak-VRAM delta MiB, ring column)}."""
    rows = {}
    with open(os.path.join(ROOT, "tests", "golden", "ring_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                ctx, delta, ring = (int(x) for x in line.split())
                rows[ctx] = (delta, ring)
    return rows


def device_memory_table(args, torch, kvd, inputs, link):
    """The shape of the [R4] Device-memory table on this machine: a 64-layer
    host-resident stack (40/8 heads, head_dim 128, bf16 GEMV stand-in) at
    4096 ... 65536 rows, ordered (depth 0) against pipelined (depth 1) per
    token, with the ring's size and the device-memory growth of each arm.  A
    128 MiB budget declines from 32768 rows on; there a larger budget (512 MiB
    at 32768, 1 GiB at 65536) engages the ring.  The ring column and the
    declines are checked against the page's table (tests/golden/ring_table.txt)."""
    from decode_attention_offloaded_amd import stack
    c = inputs.config(2)
    golden = golden_ring_table()
    plan = [(4096, ("0", "1@128")), (16384, ("0", "1@128")), (32768, ("0", "1@128", "1@512")),
            (65536, ("0", "1@128", "1@1024"))]
    out = {"layers": args.devmem_layers, "rows": {}, "checks": {}}
    for n, arms in plan:
        tokens = max(3, min(args.devmem_tokens, args.devmem_tokens * 16384 // n))
        r = stack.run_host_resident(torch, kvd, inputs, c, n_layers=args.devmem_layers, depths=arms,
                                    budget_bytes=128 << 20, tokens=tokens, warmup=2, log=log, n_rows=n,
                                    distinct_layers=4)
        frac_link(r, link)
        out["rows"][str(n)] = r
        out["checks"][str(n)] = ring_checks(n, r, golden, c.row_bytes)
        log("device memory %d rows: %s" % (n, {k: (v["ms_per_token"], v["declined"], v["ring_engaged_bytes"],
                                                    v["vram_delta_bytes"]) for k, v in r["arms"].items()}))
    return out


def ring_checks(n, res, golden, row_bytes, slack=16 << 20):
    """Against the ordered arm of the same run (the page's delta column is
    pipelined minus ordered peak memory): an engaged ring is (depth + 2) slots
    x n rows x (K + V) bytes, within its budget, grows device memory by its
    size (within `slack`: the caching allocator's own pools move by a few MiB
    between arms), and at depth 1 matches the page's ring column (decimal MB)
    within 1; a ring over its budget declines and grows nothing."""
    need1 = 3 * n * 2 * row_bytes
    base = res["arms"]["0"]["vram_delta_bytes"]
    ok, notes = True, []
    for name, arm in res["arms"].items():
        if arm["depth"] == 0:
            continue
        budget = arm["budget_bytes"]
        need = (arm["depth"] + 2) * n * 2 * row_bytes
        grow = arm["vram_delta_bytes"] - base
        if need > budget:
            good = arm["declined"] == 1 and arm["ring_engaged_bytes"] == 0 and abs(grow) <= slack
        else:
            good = (arm["declined"] == 0 and arm["ring_engaged_bytes"] == need and abs(grow - need) <= slack)
        if arm["depth"] == 1 and n in golden and arm["ring_engaged_bytes"]:
            good = good and abs(need1 / 1e6 - golden[n][1]) < 1.0
        arm["vram_growth_over_ordered_bytes"] = int(grow)
        ok = ok and good
        notes.append("%s: need %d B, budget %d B, %s, device memory over the ordered arm %+d B" % (
            name, need, budget, "declined" if arm["declined"] else "engaged %d B" % arm["ring_engaged_bytes"], grow))
    if n in golden:
        notes.append("page: ring column %d (MB), VRAM delta %d MiB; 3 x n x 2176 B = %.2f MB" % (
            golden[n][1], golden[n][0], need1 / 1e6))
    return {"ok": bool(ok), "notes": notes}


def long_context(args, torch, kvd, inputs, link):
    """131072 rows x 64 layers host-resident, whole-layer ring: depth 0/1/2 x
    budget 128 MiB / 1 GiB (depth 1 needs 816 MiB: only 1 GiB engages it;
    depth 2 needs 1088 MiB: neither does)."""
    from decode_attention_offloaded_amd import stack
    c = inputs.config(3)
    r = stack.run_host_resident(torch, kvd, inputs, c, n_layers=args.pipe_layers,
                                depths=("0", "1@128", "2@128", "1@1024", "2@1024"), budget_bytes=128 << 20,
                                tokens=args.long_tokens, warmup=2, log=log, distinct_layers=4)
    frac_link(r, link)
    r["checks"] = ring_checks(c.n_ctx, r, golden_ring_table(), c.row_bytes)
    log("long context: %s" % {k: (v["ms_per_token"], v["declined"]) for k, v in r["arms"].items()})
    return r


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
    res = {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
           "kernel": "torch.neg, %d GiB float32 read + %d GiB written, median of %d" % (gib, gib, reps)}
    # reads only, as the decode kernel's K/V stream does (kvd_hbm_read_probe)
    rd = kvd_read_ceiling(gib, reps)
    res["read_only"] = {"GBps": round(rd, 1), "frac_of_peak": round(rd / HBM_PEAK_GBS, 4),
                        "kernel": "kvd_hbm_read_probe: non-temporal 16-byte streaming reads of %d GiB, median of %d" % (gib, reps)}
    return res


def kvd_read_ceiling(gib, reps):
    from decode_attention_offloaded_amd import kvd
    return kvd.hbm_read_probe(gib << 30, reps)


def launch_floor(torch, count=64, reps=20):
    """The cost of launches alone in a replayed graph, per item: one, and two
    chained (the second reads what the first wrote, as the combine launch
    follows the decode launch), torch's elementwise negation of 20 KB (the
    size of one call's output).  Returns microseconds per item."""
    xs = [torch.ones(5120, dtype=torch.float32, device="cuda:0") for _ in range(count)]
    ys = [torch.empty_like(x) for x in xs]
    zs = [torch.empty_like(x) for x in xs]
    s = torch.cuda.Stream(device=torch.device("cuda:0"))

    def timed(body):
        with torch.cuda.stream(s):
            for i in range(count):
                body(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                body(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / (reps * count), 3)

    one = timed(lambda i: torch.neg(xs[i], out=ys[i]))
    two = timed(lambda i: (torch.neg(xs[i], out=ys[i]), torch.neg(ys[i], out=zs[i])))
    return {"one_launch_us": one, "two_chained_launches_us": two,
            "kernel": "torch.neg of 20 KB, graph-replayed over %d distinct buffers" % count}


def stream_same_bytes(torch, nbytes, reps=20, calls=64):
    """The rate a single streaming launch of one decode call's size reaches
    here: torch's elementwise negation reading nbytes / 2 and writing nbytes / 2,
    a graph of `calls` launches (as the decode calls are measured) cycling
    distinct buffers (at least 2.5 GB in all, as the decode calls cycle
    distinct layers), so launch and first-byte latency weigh as they do for a
    call.  Returns {"bytes", "us", "GBps", "frac_of_peak"}."""
    n = nbytes // 8
    count = max(4, min(64, int(2.5e9 // nbytes)))
    xs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(count)]
    ys = [torch.empty_like(x) for x in xs]
    s = torch.cuda.Stream(device=torch.device("cuda:0"))
    idx = [i % count for i in range(max(calls, count))]
    with torch.cuda.stream(s):
        for i in idx:
            torch.neg(xs[i], out=ys[i])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in idx:
            torch.neg(xs[i], out=ys[i])
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(idx))
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

def cpu_model():
    """The CPU as /proc/cpuinfo names it, with the count of sockets and of
    logical CPUs it lists."""
    names, physical, logical, ident = [], set(), 0, {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k = k.strip()
                if k == "model name":
                    names.append(v.strip())
                    logical += 1
                elif k == "physical id":
                    physical.add(v.strip())
                elif k in ("vendor_id", "cpu family", "model", "stepping", "cache size", "cpu MHz") and k not in ident:
                    ident[k] = v.strip()
    except OSError:
        pass
    model = names[0] if names else "unknown"
    return {"model_name": model, "sockets": len(physical) or None, "logical_cpus_listed": logical or None,
            "vendor": ident.get("vendor_id"), "family": ident.get("cpu family"), "model": ident.get("model"),
            "stepping": ident.get("stepping"), "cache": ident.get("cache size"), "mhz": ident.get("cpu MHz")}


def cpu_baseline(target_s=6.0):
    """The fp64 oracle on this host's cores, after the GPU legs (never beside
    them), as the plan has it: single-threaded and on every core of the
    process's affinity set, on one layer of each workload -- the 4096-row
    layer, a 16384-row layer, a 131072-row layer, and one full-attention and
    one 4096-row-window layer of the 16-sequence batch.  Median of up to 5
    timed calls after one untimed (fewer for calls over ~1 s, so the whole
    leg stays within about a minute; a call over 2 s is timed once, with no
    untimed call before it).  `value` is the 4096-row layer on every core, in
    the bench's unit."""
    import oracle
    from decode_attention_offloaded_amd import inputs
    from decode_attention_offloaded_amd.batched import cfg4_lengths
    cores = len(os.sched_getaffinity(0))
    runs = {}

    def timed(name, q, segs, hkv, d, threads, window, nbytes):
        t0 = time.perf_counter()
        oracle.attend(q, segs, hkv, d, threads=threads, window=window)
        one = time.perf_counter() - t0
        # a call over 2 s is its own measurement (no separate untimed call)
        n = 5 if one < 0.5 else 3 if one < 2.0 else 0
        ts = [one] if n == 0 else []
        for _ in range(n):
            t0 = time.perf_counter()
            oracle.attend(q, segs, hkv, d, threads=threads, window=window)
            ts.append(time.perf_counter() - t0)
        dt = float(np.median(ts))
        runs[name] = {"ms_per_layer": round(dt * 1e3, 2), "GBps": round(nbytes / dt / 1e9, 4), "threads": threads,
                      "timed_calls": len(ts), "untimed_first_call": n > 0, "bytes_per_layer": nbytes}

    work = []
    for cfg, n in ((1, 4096), (2, 16384), (3, 131072)):
        c = inputs.config(cfg)
        r = c.layer_rng(0)
        k = inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)
        v = inputs.random_kv_rows(r, n, c.n_head_kv, c.head_dim)
        q = inputs.random_q(r, 1, c.n_head_q, c.head_dim)
        work.append(("%d rows" % n, q, [[(k, v, 0)]], c, 0, algorithmic_bytes(n, c.n_head_kv, c.head_dim, c.n_head_q)))
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
    q4 = inputs.random_q(r, len(lens), c.n_head_q, c.head_dim)
    qb = 2 * len(lens) * c.n_head_q * c.head_dim * 4
    work.append(("16 sequences, full attention", q4, segs, c, 0, nb_full + qb))
    work.append(("16 sequences, 4096-row window", q4, segs, c, 4096, nb_win + qb))
    t_all = time.perf_counter()
    for threads in (1, cores):
        for name, q, sg, c, window, nbytes in work:
            timed("%s, %d thread%s" % (name, threads, "s" if threads > 1 else ""), q, sg, c.n_head_kv, c.head_dim,
                  threads, window, nbytes)
    head = runs["4096 rows, %d thread%s" % (cores, "s" if cores > 1 else "")]
    cpu = cpu_model()
    return {"value": head["GBps"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "one 4096-row, 40/8-head, head_dim-128 layer per call (fp64 oracle, OpenMP over query heads) "
                      "on %d threads, median of %d calls; the plan's other workloads and the single-thread runs are "
                      "under 'runs' (%.0f s in all); CPU: %s (family %s model %s)" % (
                          cores, head["timed_calls"], time.perf_counter() - t_all, cpu["model_name"], cpu["family"],
                          cpu["model"]),
            "ms_per_layer": head["ms_per_layer"], "cpu": cpu, "runs": runs}


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


def profile_fields(name):
    """The machine-readable fields (indented `key: value` lines) of a committed
    profile summary, or None when the kernel or plan source has changed since
    its counters were taken (or the file is missing)."""
    try:
        fields = {}
        for line in open(os.path.join(ROOT, "profiles", name)):
            if ":" in line and line.startswith("    "):
                k, v = line.strip().split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("source_sha256") == traffic_source_sha():
            return fields
    except (OSError, ValueError):
        pass
    return None


def measured_traffic():
    """HBM bytes per 4096-row call from the committed counter summary, or None."""
    f = profile_fields("decode_attention_4096rows_hbm_traffic.md")
    try:
        return int(f["traffic_bytes_per_call"]) if f else None
    except (KeyError, ValueError):
        return None


# Vector-ALU issue peak of MI355X: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64
# fp32 VALU instruction per SIMD every 4 cycles (16 lanes per SIMD; no packed
# fp32 here), in wave-instructions per second.
VALU_PEAK_GIPS = 256 * 4 * 2.4e9 / 4 / 1e9


def alu_line(us_per_call):
    """VALU instructions per 4096-row call (decode + combine, MFMA excluded),
    from the committed counter summary, against the vector-issue peak; None
    when the kernel or plan source has changed since the counters."""
    f = profile_fields("decode_attention_counters.md")
    try:
        valu = int(f["valu_wave_insts_per_call"])
        mfma = int(f["mfma_insts_per_call"])
    except (TypeError, KeyError, ValueError):
        return None
    achieved = valu / (us_per_call * 1e-6) / 1e9
    return {"bound": "alu", "achieved": round(achieved, 2), "peak": VALU_PEAK_GIPS, "unit": "G wave-instr/s",
            "frac": round(achieved / VALU_PEAK_GIPS, 4), "valu_insts_per_call": valu, "mfma_insts_per_call": mfma,
            "source": "profiles/decode_attention_counters.md (SQ_INSTS_VALU - SQ_INSTS_MFMA)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--rows", type=int, default=4096,
                    help="context of the device-resident leg (4096 = the headline workload; others for profiling)")
    ap.add_argument("--ceiling", type=int, default=1, help="measure the streaming ceiling")
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
    ap.add_argument("--long", type=int, default=1, help="run the 131072-row depth/budget sweep")
    ap.add_argument("--long-tokens", type=int, default=3)
    ap.add_argument("--devmem", type=int, default=1, help="run the device-memory table (4096 ... 65536 rows)")
    ap.add_argument("--devmem-layers", type=int, default=64)
    ap.add_argument("--devmem-tokens", type=int, default=8)
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
        "config": {"workload": "decode attention, device-resident q8_0 KV: 1 sequence x %d rows, 40 query / "
                               "8 KV heads, head_dim 128; one step = %d distinct layer caches" % (
                                   args.rows, d["layers_per_step"]),
                   "n_ctx": args.rows, "n_head_q": 40, "n_head_kv": 8, "head_dim": 128,
                   "layers_per_step": d["layers_per_step"], "kv": "q8_0 (34-byte blocks)"},
        "roofline": {"bound": "hbm", "achieved": round(d["value"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(d["value"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "decode_kernel<128,5,0,%d,%d> + combine_kernel<128> (one call; %d splits of %d "
                               "rows)" % (d["plan"]["load_mode"], d["plan"]["waves"], d["plan"]["splits"],
                                          d["plan"]["split_rows"]),
                     "bytes_per_launch": d["bytes_per_launch"], "us_per_launch": round(d["us_per_launch"], 3),
                     "alu": alu_line(d["us_per_launch"])},
        "device_curve": d["curve"],
        "hbm_stream_ceiling": hbm_stream_ceiling(torch) if args.ceiling else None,
        "calibration_copy_bytes": calib,
    }
    if args.curve and args.ceiling:
        # what one streaming launch moving a call's algorithmic bytes reaches
        c1 = inputs.config(1)
        same = {}
        for n in (4096, 16384, 32768, 131072):
            same[str(n)] = stream_same_bytes(torch, algorithmic_bytes(n, c1.n_head_kv, c1.head_dim, c1.n_head_q))
        out["hbm_stream_ceiling"]["same_bytes_as_call"] = same
        out["hbm_stream_ceiling"]["launch_floor"] = launch_floor(torch)
    log("streaming ceiling: %s" % out["hbm_stream_ceiling"])
    link = (link_peak(kvd) if (args.pipeline or args.batched or args.tiled or args.residency or args.asym
                               or args.headsplit or args.long or args.devmem) else None)
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
    if args.devmem:
        out["device_memory_table"] = device_memory_table(args, torch, kvd, inputs, link)
    if args.long:
        out["long_context"] = long_context(args, torch, kvd, inputs, link)
    if args.cpu_baseline:
        # after every GPU leg, so the oracle never competes with DMA for host memory
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
