"""Per-head residency split of a host-resident stack ("F5 — Advanced KV Cache
Techniques", M2 HeadInfer: a fraction of the KV heads stays resident on the
device, the rest lives in host memory and is brought back for every attention
step; the split is on whole KV heads, so every query group stays with its KV
head).

Here KV heads [0, hr) of every layer stay on the device and heads [hr, H)
are packed per layer in pinned host memory ((H - hr) chunks per row) and
staged through the ring one layer ahead.  Attention runs as two calls per
layer over disjoint head ranges -- the resident heads from device memory, the
staged heads from the ring's view -- writing disjoint query-head ranges of the
output, so no merge is needed (the reassembly on the head axis is just where
each call writes).  Only the residency is split: every head's attention runs
on the GPU (the pages defer the compute split, and attention of host-resident
heads on the host is not part of this library).
"""
from __future__ import annotations

import time
from typing import Optional

import numpy as np

from decode_attention_offloaded_amd.stack import PinnedBuffer, cfg_q


class HeadSplitKV:
    """K/V of a stack split by KV head: device [L][n][hr*CB], pinned host [L][n][(H-hr)*CB]."""

    def __init__(self, torch, inputs, cfg, n_layers: int, n_rows: int, hr: int, distinct: Optional[int] = None):
        H = cfg.n_head_kv
        if not 0 <= hr <= H:
            raise ValueError("resident heads must be in [0, n_head_kv]")
        self.n_layers, self.n_rows, self.hr, self.H = n_layers, n_rows, hr, H
        self.cb = cfg.head_dim // 32 * 34
        self.dev_bytes, self.host_bytes = hr * self.cb, (H - hr) * self.cb
        dev = torch.device("cuda:0")
        distinct = n_layers if distinct is None else max(1, min(distinct, n_layers))
        lb = n_rows * self.host_bytes
        self.k = PinnedBuffer(max(1, n_layers * lb))
        self.v = PinnedBuffer(max(1, n_layers * lb))
        self.layer_host_bytes = lb
        self.dev_k, self.dev_v = [], []
        for l in range(n_layers):
            if l < distinct:
                r = cfg.layer_rng(l)
                k = inputs.random_kv_rows(r, n_rows, H, cfg.head_dim)
                v = inputs.random_kv_rows(r, n_rows, H, cfg.head_dim)
                self.host_k(l)[:] = k[:, self.dev_bytes:]
                self.host_v(l)[:] = v[:, self.dev_bytes:]
                self.dev_k.append(torch.from_numpy(np.ascontiguousarray(k[:, :self.dev_bytes])).to(dev))
                self.dev_v.append(torch.from_numpy(np.ascontiguousarray(v[:, :self.dev_bytes])).to(dev))
            else:
                src = l % distinct
                self.host_k(l)[:] = self.host_k(src)
                self.host_v(l)[:] = self.host_v(src)
                self.dev_k.append(self.dev_k[src])
                self.dev_v.append(self.dev_v[src])

    def host_k(self, l):
        o = l * self.layer_host_bytes
        return self.k.array[o:o + self.layer_host_bytes].reshape(self.n_rows, self.host_bytes)

    def host_v(self, l):
        o = l * self.layer_host_bytes
        return self.v.array[o:o + self.layer_host_bytes].reshape(self.n_rows, self.host_bytes)

    def full_rows(self, l):
        """Whole K and V rows of layer l (device part + host part) as numpy, for checks."""
        k = np.concatenate([self.dev_k[l].cpu().numpy(), self.host_k(l)], axis=1)
        v = np.concatenate([self.dev_v[l].cpu().numpy(), self.host_v(l)], axis=1)
        return k, v

    def free(self):
        self.k.free()
        self.v.free()
        self.dev_k = self.dev_v = None


class HeadSplitStack:
    """One arm (ring depth and budget) over a HeadSplitKV, one decode token at a time."""

    def __init__(self, torch, kvd, cfg, kv: HeadSplitKV, depth: int, budget_bytes: int, gemv_weights=None,
                 stream=None, pool: int = 4):
        self.torch, self.kvd, self.cfg, self.kv = torch, kvd, cfg, kv
        self.depth = depth
        dev = torch.device("cuda:0")
        self.stream = stream or torch.cuda.Stream(device=dev)
        self.ring = kvd.Ring(depth, budget_bytes)
        hb = max(kv.host_bytes, 4)
        self.ordered_k = torch.empty(kv.n_rows * hb, dtype=torch.uint8, device=dev)
        self.ordered_v = torch.empty(kv.n_rows * hb, dtype=torch.uint8, device=dev)
        g = np.random.default_rng([cfg.seed, 7777])
        self.q = [torch.from_numpy(cfg_q(g, cfg)).to(dev) for _ in range(kv.n_layers)]
        self.out = [torch.empty_like(self.q[0]) for _ in range(kv.n_layers)]
        self.ws = kvd.Workspace()
        self.gemv = gemv_weights
        if gemv_weights is not None:
            self.x = torch.randn(1, gemv_weights[0].shape[0], dtype=torch.bfloat16, device=dev,
                                 generator=torch.Generator(device=dev).manual_seed(cfg.seed))
            self.y = torch.empty(1, gemv_weights[0].shape[1], dtype=torch.bfloat16, device=dev)
        from decode_attention_offloaded_amd import inputs
        gp = np.random.default_rng([cfg.seed, 4242])
        rows = [(inputs.random_kv_rows(gp, 1, cfg.n_head_kv, cfg.head_dim)[0],
                 inputs.random_kv_rows(gp, 1, cfg.n_head_kv, cfg.head_dim)[0]) for _ in range(pool)]
        d = kv.dev_bytes
        self.pool_host = [(k[d:].copy(), v[d:].copy()) for k, v in rows]
        self.pool_dev = [(torch.from_numpy(k[:d].copy()).to(dev), torch.from_numpy(v[:d].copy()).to(dev))
                         for k, v in rows]
        G = cfg.n_head_q // cfg.n_head_kv
        self.gq = G * kv.hr   # query heads served by the resident KV heads

    def _stage(self, l, flags):
        kv = self.kv
        o = l * kv.layer_host_bytes
        n = kv.n_rows
        return self.ring.stage(l, flags, kv.k.ptr + o, kv.v.ptr + o, kv.host_bytes, n, n - 1, n,
                               self.ordered_k.data_ptr(), self.ordered_v.data_ptr(), stream=self.stream)

    def token(self, t: int):
        """One decode token over every layer; returns its time in ms (compute-stream events)."""
        torch, kvd, kv = self.torch, self.kvd, self.kv
        L, N, s, n = kv.n_layers, self.depth, self.stream, kv.n_rows
        staged = kv.hr < kv.H
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            if staged:
                for l in range(min(N, L)):
                    self._stage(l, kvd.STAGE_PREFETCH)
            for l in range(L):
                if self.gemv is not None:
                    torch.matmul(self.x, self.gemv[l % len(self.gemv)], out=self.y)
                p = (t * 7 + l) % len(self.pool_dev)
                # the newest row: its resident heads on the device, the rest on the host
                if kv.hr:
                    kv.dev_k[l][n - 1].copy_(self.pool_dev[p][0])
                    kv.dev_v[l][n - 1].copy_(self.pool_dev[p][1])
                    kvd.attend_decode(self.q[l][:, :self.gq], self.out[l][:, :self.gq],
                                      [[(kv.dev_k[l], kv.dev_v[l], 0)]], kv.hr, workspace=self.ws, stream=s)
                if staged:
                    kv.host_k(l)[n - 1] = self.pool_host[p][0]
                    kv.host_v(l)[n - 1] = self.pool_host[p][1]
                    _, view = self._stage(l, kvd.STAGE_ACQUIRE)
                    kvd.attend_decode(self.q[l][:, self.gq:], self.out[l][:, self.gq:],
                                      [[(view.k, view.v, view.n_rows, 0, view.row_stride)]], kv.H - kv.hr,
                                      workspace=self.ws, stream=s)
                    self.ring.release(l, stream=s)
                    if N > 0 and l + N < L:
                        self._stage(l + N, kvd.STAGE_PREFETCH)
            e1.record(s)
        s.synchronize()
        return e0.elapsed_time(e1)

    def close(self):
        self.stream.synchronize()
        self.ring.close()
        self.ring = None


def run_headsplit(torch, kvd, inputs, cfg, resident_heads: int, n_layers=64, depths=(0, 1), budget_bytes=1 << 30,
                  tokens=3, warmup=1, log=print, n_rows=None, gemv=True, distinct_layers=None, check=None):
    """Ordered vs pipelined per-token time with KV heads [0, resident_heads)
    device-resident and the rest staged, arms A/B/B/A.  check(stack, kv) runs on
    the last arm.  Returns a dict for the benchmark."""
    n_rows = n_rows or cfg.n_ctx
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    kv = HeadSplitKV(torch, inputs, cfg, n_layers, n_rows, resident_heads, distinct=distinct_layers)
    log("head split: %d of %d KV heads resident, %d layers x %d rows, %.2f GB pinned, set up in %.1f s" %
        (resident_heads, cfg.n_head_kv, n_layers, n_rows, 2 * kv.k.nbytes / 1e9, time.perf_counter() - t0))
    weights = None
    if gemv:
        gen = torch.Generator(device=dev).manual_seed(cfg.seed)
        m, n = cfg.extra.get("gemv", (5120, 27648))
        weights = [(torch.randn(m, n, dtype=torch.bfloat16, device=dev, generator=gen) * 0.02)
                   for _ in range(n_layers)]
    order = list(depths) + list(reversed(depths))
    compute = torch.cuda.Stream(device=dev)
    times = {d: [] for d in depths}
    outs, stats = {}, {}
    for i, d in enumerate(order):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        st = HeadSplitStack(torch, kvd, cfg, kv, d, budget_bytes, gemv_weights=weights, stream=compute)
        for t in range(warmup):
            st.token(t)
        for t in range(warmup, warmup + tokens):
            times[d].append(st.token(t))
        outs[d] = [o.clone() for o in st.out]
        stats[d] = st.ring.stats()
        if check is not None and i == len(order) - 1:
            check(st, kv)
        st.close()
        del st
        torch.cuda.empty_cache()
    identical = all(torch.equal(a, b) for a, b in zip(outs[depths[0]], outs[depths[-1]]))
    staged = 2 * n_layers * n_rows * kv.host_bytes
    res = {"n_ctx": n_rows, "n_layers": n_layers, "resident_heads": resident_heads, "n_head_kv": cfg.n_head_kv,
           "resident_bytes": 2 * n_layers * n_rows * kv.dev_bytes, "staged_bytes_per_token": staged,
           "tokens_timed": tokens, "order": order, "bit_identical": bool(identical), "arms": {}}
    for d in depths:
        ms = float(np.median(times[d]))
        s = stats[d]
        res["arms"][str(d)] = {"depth": d, "ms_per_token": round(ms, 3),
                               "staged_GBps": round(staged / (ms * 1e-3) / 1e9, 2),
                               "ring_engaged_bytes": s["ring_bytes"] if s["engaged"] else 0,
                               "declined": s["declined"], "n_acquire_pipelined": s["n_acquire_pipelined"],
                               "n_acquire_ordered": s["n_acquire_ordered"]}
    kv.free()
    del weights
    torch.cuda.empty_cache()
    return res
