"""A host-resident decode stack driven through the staging ring.

This is the caller side of the ring ABI, used by the benchmark and the GPU
tests: a stack of layers whose q8_0 K/V live in pinned host memory, one decode
token at a time.  Per token and layer l (following "sched: pipeline the
delivery of a host-resident KV cache (R4)", What it does):
    stand-in compute (bf16 GEMV) on the compute stream;
    the host writes layer l's newest row (the only row the step writes, so
    the stable prefix is every older row);
    ACQUIRE l -> a device view (ordered copy, or pipelined slot + tail);
    decode attention on the view;
    RELEASE l; PREFETCH l + N (the next delivery is issued after this layer's
    consumer is enqueued).
The first N layers of a token are prefetched at the token start, and the
token ends with a synchronisation of the compute stream (where a sampler would
read the logits).
"""
from __future__ import annotations

import ctypes
import time
from typing import Callable, Optional

import numpy as np


class PinnedBuffer:
    """hipHostMalloc'ed host memory as a numpy uint8 array (exact size, no rounding)."""

    _hip = None

    def __init__(self, nbytes: int):
        import torch  # noqa: F401  (load torch's HIP runtime: one runtime per process)
        if PinnedBuffer._hip is None:
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipHostMalloc.restype = ctypes.c_int
            h.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
            h.hipHostFree.restype = ctypes.c_int
            h.hipHostFree.argtypes = [ctypes.c_void_p]
            PinnedBuffer._hip = h
        p = ctypes.c_void_p()
        rc = PinnedBuffer._hip.hipHostMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes), 0)
        if rc != 0 or not p.value:
            raise MemoryError("hipHostMalloc(%d) failed: %d" % (nbytes, rc))
        self.ptr = p.value
        self.nbytes = nbytes
        self.array = np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(self.ptr))

    def free(self):
        if self.ptr:
            self.array = None
            PinnedBuffer._hip.hipHostFree(ctypes.c_void_p(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class HostKV:
    """K and V of n_layers layers, each [cap_rows][row_bytes] (V rows v_row_bytes
    wide: shorter for a q4_0 V cache), in pinned host memory."""

    def __init__(self, n_layers: int, cap_rows: int, row_bytes: int, v_row_bytes: Optional[int] = None,
                 v_type: int = 0):
        self.n_layers, self.cap_rows, self.row_bytes = n_layers, cap_rows, row_bytes
        self.v_row_bytes = v_row_bytes or row_bytes
        self.v_type = v_type
        self.layer_bytes = cap_rows * row_bytes
        self.v_layer_bytes = cap_rows * self.v_row_bytes
        self.k = PinnedBuffer(n_layers * self.layer_bytes)
        self.v = PinnedBuffer(n_layers * self.v_layer_bytes)

    def k_rows(self, layer):
        o = layer * self.layer_bytes
        return self.k.array[o:o + self.layer_bytes].reshape(self.cap_rows, self.row_bytes)

    def v_rows(self, layer):
        o = layer * self.v_layer_bytes
        return self.v.array[o:o + self.v_layer_bytes].reshape(self.cap_rows, self.v_row_bytes)

    def k_ptr(self, layer):
        return self.k.ptr + layer * self.layer_bytes

    def v_ptr(self, layer):
        return self.v.ptr + layer * self.v_layer_bytes

    def fill(self, inputs, cfg, n_rows: int, distinct: Optional[int] = None):
        """Seeded q8_0 K rows and q8_0 (or q4_0) V rows.  With `distinct`, only that
        many layers are drawn and the rest repeat them (keeps very large stacks
        quick to set up)."""
        distinct = self.n_layers if distinct is None else min(distinct, self.n_layers)
        vgen = inputs.random_kv_rows_q4_0 if self.v_type == 1 else inputs.random_kv_rows
        for l in range(self.n_layers):
            if l < distinct:
                r = cfg.layer_rng(l)
                self.k_rows(l)[:n_rows] = inputs.random_kv_rows(r, n_rows, cfg.n_head_kv, cfg.head_dim)
                self.v_rows(l)[:n_rows] = vgen(r, n_rows, cfg.n_head_kv, cfg.head_dim)
            else:
                self.k_rows(l)[:n_rows] = self.k_rows(l % distinct)[:n_rows]
                self.v_rows(l)[:n_rows] = self.v_rows(l % distinct)[:n_rows]

    def free(self):
        self.k.free()
        self.v.free()


class Stack:
    """Drives one arm (a ring of some depth and budget) over a HostKV."""

    def __init__(self, torch, kvd, cfg, host: HostKV, n_rows: int, depth: int, budget_bytes: int,
                 gemv_weights=None, stream=None, new_rows=None, resident: int = 0, cross_step: bool = False):
        self.torch, self.kvd, self.cfg, self.host = torch, kvd, cfg, host
        self.n_rows, self.depth = n_rows, depth
        dev = torch.device("cuda:0")
        # layers [0, resident) keep their K/V on the device (a resident
        # prefix); the rest are staged through the ring each step
        self.resident = max(0, min(int(resident), host.n_layers))
        # cross-step look-ahead: after the last layer of a step, the first N
        # staged layers of the next step are prefetched (their prefix is
        # stable: a step rewrites only the newest row), so the next step does
        # not start with an exposed delivery
        self.cross_step = cross_step
        self._primed = set()
        self.dev_k = [torch.from_numpy(host.k_rows(l)[:n_rows]).to(dev) for l in range(self.resident)]
        self.dev_v = [torch.from_numpy(host.v_rows(l)[:n_rows]).to(dev) for l in range(self.resident)]
        self.pool_dev = None
        if self.resident and new_rows is not None and hasattr(new_rows, "rows"):
            self.pool_dev = [(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)) for k, v in new_rows.rows]
        self.stream = stream or torch.cuda.Stream(device=dev)
        self.ring = kvd.Ring(depth, budget_bytes)
        rb = host.row_bytes
        self.ordered_k = torch.empty(host.cap_rows * rb, dtype=torch.uint8, device=dev)
        self.ordered_v = torch.empty(host.cap_rows * host.v_row_bytes, dtype=torch.uint8, device=dev)
        g = np.random.default_rng([cfg.seed, 7777])
        self.q = [torch.from_numpy(cfg_q(g, cfg)).to(dev) for _ in range(host.n_layers)]
        self.out = [torch.empty_like(self.q[0]) for _ in range(host.n_layers)]
        self.ws = kvd.Workspace()
        self.gemv = gemv_weights
        if gemv_weights is not None:
            self.x = torch.randn(1, gemv_weights[0].shape[0], dtype=torch.bfloat16, device=dev,
                                 generator=torch.Generator(device=dev).manual_seed(cfg.seed))
            self.y = torch.empty(1, gemv_weights[0].shape[1], dtype=torch.bfloat16, device=dev)
        self.new_rows = new_rows  # callable(token, layer) -> (k_row, v_row) bytes, or None
        self.on_view: Optional[Callable] = None  # test hook: (layer, view) after ACQUIRE
        self.after_attend: Optional[Callable] = None  # test hook: (layer, view) before RELEASE

    def _stage(self, layer, flags):
        h = self.host
        return self.ring.stage(layer, flags, h.k_ptr(layer), h.v_ptr(layer), h.row_bytes, self.n_rows,
                               self.n_rows - 1, h.cap_rows, self.ordered_k.data_ptr(), self.ordered_v.data_ptr(),
                               stream=self.stream, v_row_bytes=h.v_row_bytes)

    def token(self, t: int):
        """One decode token over every layer; returns the token time in ms (compute-stream events)."""
        torch, kvd, h = self.torch, self.kvd, self.host
        L, N, s = h.n_layers, self.depth, self.stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        R = self.resident
        with torch.cuda.stream(s):
            e0.record(s)
            for l in range(R, min(R + N, L)):
                if l not in self._primed:
                    self._stage(l, kvd.STAGE_PREFETCH)
            self._primed = set()
            for l in range(L):
                if self.gemv is not None:
                    torch.matmul(self.x, self.gemv[l % len(self.gemv)], out=self.y)
                if self.new_rows is not None:
                    kr, vr = self.new_rows(t, l)
                    h.k_rows(l)[self.n_rows - 1] = kr
                    h.v_rows(l)[self.n_rows - 1] = vr
                if l < R:
                    # resident layer: the newest row is written on the device
                    if self.new_rows is not None:
                        if self.pool_dev is not None:
                            kd, vd = self.pool_dev[self.new_rows.index(t, l)]
                        else:
                            kd, vd = torch.from_numpy(kr).to(s.device), torch.from_numpy(vr).to(s.device)
                        self.dev_k[l][self.n_rows - 1].copy_(kd)
                        self.dev_v[l][self.n_rows - 1].copy_(vd)
                    kvd.attend_decode(self.q[l], self.out[l], [[(self.dev_k[l], self.dev_v[l], 0)]],
                                      self.cfg.n_head_kv, workspace=self.ws, stream=s, v_type=h.v_type)
                    continue
                rc, view = self._stage(l, kvd.STAGE_ACQUIRE)
                if self.on_view is not None:
                    self.on_view(l, view)
                kvd.attend_decode(self.q[l], self.out[l],
                                  [[(view.k, view.v, view.n_rows, 0, view.row_stride, view.v_row_stride)]],
                                  self.cfg.n_head_kv, workspace=self.ws, stream=s, v_type=h.v_type)
                if self.after_attend is not None:
                    self.after_attend(l, view)
                self.ring.release(l, stream=s)
                if l + N < L and N > 0 and l + N >= R + N:
                    self._stage(l + N, kvd.STAGE_PREFETCH)
            if self.cross_step and N > 0:
                for l in range(R, min(R + N, L)):
                    rc, _ = self._stage(l, kvd.STAGE_PREFETCH)
                    if rc == kvd.KVD_OK:
                        self._primed.add(l)
            e1.record(s)
        s.synchronize()
        return e0.elapsed_time(e1)

    def close(self):
        self.stream.synchronize()
        self.ring.close()
        self.ring = None


def cfg_q(g, cfg):
    return g.standard_normal((1, cfg.n_head_q, cfg.head_dim)).astype(np.float32)


def token_rows(cfg, pool: int = 4, v_type: int = 0):
    """A callable giving the newest K/V row written at (token, layer): a small
    seeded pool, so the host loop does no random drawing while timed."""
    from decode_attention_offloaded_amd import inputs
    g = np.random.default_rng([cfg.seed, 4242])
    vgen = inputs.random_kv_rows_q4_0 if v_type == 1 else inputs.random_kv_rows
    rows = [(inputs.random_kv_rows(g, 1, cfg.n_head_kv, cfg.head_dim)[0],
             vgen(g, 1, cfg.n_head_kv, cfg.head_dim)[0]) for _ in range(pool * 7)]

    def index(t, l):
        return (t * 7 + l) % len(rows)

    def f(t, l):
        return rows[index(t, l)]
    f.rows, f.index = rows, index
    return f


def run_host_resident(torch, kvd, inputs, cfg, n_layers=64, depths=(0, 1), budget_bytes=128 << 20, tokens=8,
                      warmup=3, log=print, n_rows=None, gemv=True, distinct_layers=None, v_type=0,
                      cross_step=False):
    """Ordered vs pipelined per-token time for a host-resident stack, arms run
    A/B/B/A (reversed order on the second pass).  Returns a dict for the bench."""
    n_rows = n_rows or cfg.n_ctx
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    vrb = inputs.row_bytes_q4_0(cfg.n_head_kv, cfg.head_dim) if v_type == 1 else cfg.row_bytes
    host = HostKV(n_layers, n_rows, cfg.row_bytes, vrb, v_type)
    host.fill(inputs, cfg, n_rows, distinct=distinct_layers)
    log("host KV: %d layers x %d rows, %.2f GB pinned, filled in %.1f s" %
        (n_layers, n_rows, (host.k.nbytes + host.v.nbytes) / 1e9, time.perf_counter() - t0))
    weights = None
    if gemv:
        gen = torch.Generator(device=dev).manual_seed(cfg.seed)
        m, n = cfg.extra.get("gemv", (5120, 27648))
        weights = [(torch.randn(m, n, dtype=torch.bfloat16, device=dev, generator=gen) * 0.02)
                   for _ in range(n_layers)]
    rows_fn = token_rows(cfg, v_type=v_type)
    # an arm is a depth, "<depth>x" for that depth with cross-step look-ahead,
    # or "<depth>@<MiB>" for that depth under its own budget
    arm_budget = {d: (int(str(d).split("@")[1]) << 20 if "@" in str(d) else budget_bytes) for d in depths}
    order = list(depths) + list(reversed(depths))
    # One compute stream for every arm, as an engine has one: streams share the
    # process's few hardware queues, and a fresh stream per arm would make the
    # queue a transfer stream lands on (and so the overlap) vary between arms.
    compute = torch.cuda.Stream(device=dev)
    times = {d: [] for d in depths}
    outs, stats, vram = {}, {}, {}
    for d in order:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        free0 = torch.cuda.mem_get_info(dev)[0]
        depth, cross = int(str(d).split("@")[0].rstrip("x")), cross_step or str(d).endswith("x")
        st = Stack(torch, kvd, cfg, host, n_rows, depth, arm_budget[d], gemv_weights=weights, new_rows=rows_fn,
                   stream=compute, cross_step=cross)
        for t in range(warmup):
            st.token(t)
        free1 = torch.cuda.mem_get_info(dev)[0]
        for t in range(warmup, warmup + tokens):
            times[d].append(st.token(t))
        outs[d] = [o.clone() for o in st.out]
        stats[d] = st.ring.stats()
        vram[d] = free0 - free1
        st.close()
        del st
        torch.cuda.empty_cache()
    identical = all(torch.equal(a, b) for d in depths[1:] for a, b in zip(outs[depths[0]], outs[d]))
    bytes_token = n_layers * n_rows * (cfg.row_bytes + vrb)
    res = {"n_ctx": n_rows, "n_layers": n_layers, "tokens_timed": tokens, "order": order, "v_type": v_type,
           "bytes_per_token": bytes_token, "bit_identical": bool(identical), "arms": {}}
    for d in depths:
        ms = float(np.median(times[d]))
        s = stats[d]
        res["arms"][str(d)] = {"depth": int(str(d).split("@")[0].rstrip("x")),
                               "cross_step": cross_step or str(d).endswith("x"), "budget_bytes": arm_budget[d],
                               "ms_per_token": round(ms, 3), "tokens_per_s": round(1e3 / ms, 3),
                               "staged_GBps": round(bytes_token / (ms * 1e-3) / 1e9, 2),
                               "ring_engaged_bytes": s["ring_bytes"] if s["engaged"] else 0,
                               "need_bytes": s["need_bytes"], "declined": s["declined"],
                               "vram_delta_bytes": int(vram[d]),
                               "n_prefetch": s["n_prefetch"], "n_acquire_pipelined": s["n_acquire_pipelined"],
                               "n_acquire_ordered": s["n_acquire_ordered"], "bytes_early": s["bytes_early"],
                               "bytes_late": s["bytes_late"]}
    host.free()
    del weights
    torch.cuda.empty_cache()
    return res


def run_residency(torch, kvd, inputs, cfg, arms, n_layers=64, tokens=3, warmup=1, log=print, n_rows=None,
                  distinct_layers=None, host=None):
    """Per-token time of several residency arms over one host stack, A/B/B/A.

    arms: list of (name, depth, budget_bytes, resident).  Each arm keeps layers
    [0, resident) on the device and stages the rest (ring of `depth` within
    `budget_bytes`, or ordered).  Outputs of every arm must agree bit for bit:
    attention reads the same bytes whichever memory holds them."""
    n_rows = n_rows or cfg.n_ctx
    dev = torch.device("cuda:0")
    own = host is None
    if own:
        t0 = time.perf_counter()
        host = HostKV(n_layers, n_rows, cfg.row_bytes)
        host.fill(inputs, cfg, n_rows, distinct=distinct_layers)
        log("host KV: %d layers x %d rows, %.2f GB pinned, filled in %.1f s" %
            (n_layers, n_rows, 2 * host.k.nbytes / 1e9, time.perf_counter() - t0))
    gen = torch.Generator(device=dev).manual_seed(cfg.seed)
    m, n = cfg.extra.get("gemv", (5120, 27648))
    weights = [(torch.randn(m, n, dtype=torch.bfloat16, device=dev, generator=gen) * 0.02) for _ in range(n_layers)]
    rows_fn = token_rows(cfg)
    compute = torch.cuda.Stream(device=dev)
    order = list(range(len(arms))) + list(reversed(range(len(arms))))
    times = {i: [] for i in range(len(arms))}
    outs, stats = {}, {}
    for i in order:
        name, depth, budget, resident = arms[i]
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        st = Stack(torch, kvd, cfg, host, n_rows, depth, budget, gemv_weights=weights, new_rows=rows_fn,
                   stream=compute, resident=resident)
        for t in range(warmup):
            st.token(t)
        for t in range(warmup, warmup + tokens):
            times[i].append(st.token(t))
        outs[i] = [o.clone() for o in st.out]
        stats[i] = st.ring.stats()
        st.close()
        del st
        torch.cuda.empty_cache()
    identical = all(torch.equal(a, b) for j in range(1, len(arms)) for a, b in zip(outs[0], outs[j]))
    res = {"n_ctx": n_rows, "n_layers": n_layers, "tokens_timed": tokens, "bit_identical": bool(identical),
           "arms": {}}
    for i, (name, depth, budget, resident) in enumerate(arms):
        ms = float(np.median(times[i]))
        s = stats[i]
        staged = 2 * (n_layers - resident) * n_rows * cfg.row_bytes
        res["arms"][name] = {"depth": depth, "budget_bytes": budget, "resident_layers": resident,
                             "ms_per_token": round(ms, 3), "staged_bytes_per_token": staged,
                             "staged_GBps": round(staged / (ms * 1e-3) / 1e9, 2),
                             "ring_engaged_bytes": s["ring_bytes"] if s["engaged"] else 0,
                             "declined": s["declined"], "n_acquire_pipelined": s["n_acquire_pipelined"],
                             "n_acquire_ordered": s["n_acquire_ordered"]}
    if own:
        host.free()
    del weights
    torch.cuda.empty_cache()
    return res
