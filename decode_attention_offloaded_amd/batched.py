"""Batched variable-length decode with sliding-window layers and two residency
segments per sequence, driven through the staging ring.

The caller side of the library for a batch of sequences whose older rows live
in pinned host memory and whose newer rows live on the device.  Readings
(each restates a passage in our own words):

* Which rows are host-resident: the older half of each sequence's rows,
  [0, n // 2); the newer half, which holds the newest row, stays on the
  device.  (The pages split one attention between host-held and device-held
  KV by heads, "F5 — Advanced KV Cache Techniques", M2/M3; the batched
  workload here splits by rows, and the two parts meet in the same merge.)
* The host rows of one layer are packed sequence-major into one per-layer host
  range, so the ring stages them as one contiguous delivery ("sched: pipeline
  the delivery of a host-resident KV cache (R4)", What it does: deliveries are
  contiguous byte ranges of a stable prefix).
* Sliding-window layers (odd layers; model-native sliding-window attention,
  "Plan: lossless long context ...", llama — sparse attention parity
  boundary) stage only the host rows inside the window of the sequence's
  query: a row at position p is visible from the query at position P iff
  0 <= P - p < W.  Rows outside the window are never copied.
* Older rows do not change during decode (the step writes only the newest row,
  which is device-resident), so the whole packed range is a stable prefix and
  no tail is ever copied.
* The two segments of a sequence (staged older rows, device newer rows) are
  merged by the online-softmax combine that merges splits ("F5 — Advanced KV
  Cache Techniques", M4: partial attentions merged by their maxima and sums).

Per token and layer: stand-in compute (one bf16 GEMM over the batch), the
newest row of every sequence written on the device, ACQUIRE of the packed
host range (skipped when it is empty), attention over the two segments,
RELEASE, PREFETCH of the layer N ahead.
"""
from __future__ import annotations

import time
from typing import Optional

import numpy as np

from decode_attention_offloaded_amd.stack import PinnedBuffer


class BatchedLayout:
    """Row bookkeeping of the batch: which rows are staged, where they sit.

    lengths : int array [n_seq], rows of each sequence (the query is at n - 1).
    window  : W of the sliding-window layers (odd layers); 0 disables them.
    """

    def __init__(self, lengths, n_layers: int, window: int, row_bytes: int):
        self.n = np.asarray(lengths, dtype=np.int64)
        if self.n.ndim != 1 or len(self.n) < 1 or (self.n < 2).any():
            raise ValueError("every sequence needs at least 2 rows")
        self.n_seq, self.n_layers, self.row_bytes = len(self.n), int(n_layers), int(row_bytes)
        self.h = self.n // 2                      # host rows [0, h), device rows [h, n)
        self.q_pos = self.n - 1
        self.dev_rows = self.n - self.h
        self.dev_off = np.concatenate([[0], np.cumsum(self.dev_rows)[:-1]])
        self.dev_total = int(self.dev_rows.sum())
        self.window = [window if (window > 0 and l % 2 == 1) else 0 for l in range(n_layers)]
        self.lo, self.stage_rows, self.stage_off, self.stage_total = [], [], [], []
        for l in range(n_layers):
            w = self.window[l]
            lo = np.zeros_like(self.n) if w == 0 else np.minimum(np.maximum(0, self.q_pos - w + 1), self.h)
            rows = self.h - lo
            self.lo.append(lo)
            self.stage_rows.append(rows)
            self.stage_off.append(np.concatenate([[0], np.cumsum(rows)[:-1]]))
            self.stage_total.append(int(rows.sum()))
        self.cap_rows = max(max(self.stage_total), 1)
        self.host_layer_off = np.concatenate([[0], np.cumsum(self.stage_total)[:-1]]) * self.row_bytes
        self.host_bytes = int(sum(self.stage_total)) * self.row_bytes

    def staged_bytes_per_token(self) -> int:
        """K + V bytes delivered from the host per token (every layer's packed range)."""
        return 2 * int(sum(self.stage_total)) * self.row_bytes

    def visible_bytes_per_token(self) -> int:
        """K + V bytes of the rows attention reads per token (both segments)."""
        tot = 0
        for l in range(self.n_layers):
            w = self.window[l]
            vis = self.n if w == 0 else np.minimum(self.n, w)
            tot += int(vis.sum())
        return 2 * tot * self.row_bytes


def cfg4_lengths(cfg, n_seq: Optional[int] = None, median: Optional[int] = None, lo: int = 1024, hi: int = 32768):
    from decode_attention_offloaded_amd import inputs
    g = np.random.default_rng([cfg.seed, 31337])
    return inputs.lognormal_lengths(g, n_seq or cfg.n_seq, median=median or cfg.n_ctx, sigma=1.0, lo=lo, hi=hi)


class BatchedKV:
    """Seeded K/V of the batch: packed host ranges (pinned) and device halves.

    With `distinct`, only that many layers are drawn and the rest repeat them
    (host bytes are copied, device halves are shared), which keeps a 64-layer
    stack quick to set up.
    """

    def __init__(self, torch, inputs, cfg, layout: BatchedLayout, distinct: Optional[int] = None):
        self.layout = lay = layout
        rb = lay.row_bytes
        self.k = PinnedBuffer(max(lay.host_bytes, 1))
        self.v = PinnedBuffer(max(lay.host_bytes, 1))
        dev = torch.device("cuda:0")
        distinct = lay.n_layers if distinct is None else max(1, min(distinct, lay.n_layers))
        self.dev_k, self.dev_v = [], []
        for l in range(lay.n_layers):
            hk, hv = self.host_rows(l)
            if l < distinct:
                r = cfg.layer_rng(l)
                # host rows first (sequence-major), then the device halves
                for s in range(lay.n_seq):
                    n = int(lay.stage_rows[l][s])
                    o = int(lay.stage_off[l][s])
                    if n:
                        hk[o:o + n] = inputs.random_kv_rows(r, n, cfg.n_head_kv, cfg.head_dim)
                        hv[o:o + n] = inputs.random_kv_rows(r, n, cfg.n_head_kv, cfg.head_dim)
                dk = inputs.random_kv_rows(r, lay.dev_total, cfg.n_head_kv, cfg.head_dim)
                dv = inputs.random_kv_rows(r, lay.dev_total, cfg.n_head_kv, cfg.head_dim)
                self.dev_k.append(torch.from_numpy(dk).to(dev))
                self.dev_v.append(torch.from_numpy(dv).to(dev))
            else:
                src = l % distinct
                sk, sv = self.host_rows(src)
                # same parity => same window => same packed geometry; otherwise copy per sequence
                for s in range(lay.n_seq):
                    n = int(lay.stage_rows[l][s])
                    if not n:
                        continue
                    o = int(lay.stage_off[l][s])
                    # rows [lo, h) of layer l are rows [lo - lo_src, h - lo_src) of layer src's packed range
                    o_src = int(lay.stage_off[src][s]) + int(lay.lo[l][s] - lay.lo[src][s])
                    if lay.lo[l][s] >= lay.lo[src][s]:
                        hk[o:o + n] = sk[o_src:o_src + n]
                        hv[o:o + n] = sv[o_src:o_src + n]
                    else:  # src is a window layer with fewer rows: draw the rest
                        r = np.random.default_rng([cfg.seed, l, s])
                        hk[o:o + n] = inputs.random_kv_rows(r, n, cfg.n_head_kv, cfg.head_dim)
                        hv[o:o + n] = inputs.random_kv_rows(r, n, cfg.n_head_kv, cfg.head_dim)
                self.dev_k.append(self.dev_k[src])
                self.dev_v.append(self.dev_v[src])

    def host_rows(self, l):
        lay = self.layout
        o, n = int(lay.host_layer_off[l]), lay.stage_total[l] * lay.row_bytes
        return (self.k.array[o:o + n].reshape(-1, lay.row_bytes), self.v.array[o:o + n].reshape(-1, lay.row_bytes))

    def host_ptrs(self, l):
        o = int(self.layout.host_layer_off[l])
        return self.k.ptr + o, self.v.ptr + o

    def oracle_segments(self, l):
        """Per sequence [(host K, host V, pos0), (device K, device V, pos0)] as numpy arrays."""
        lay = self.layout
        hk, hv = self.host_rows(l)
        dk, dv = self.dev_k[l].cpu().numpy(), self.dev_v[l].cpu().numpy()
        segs = []
        for s in range(lay.n_seq):
            o, n = int(lay.stage_off[l][s]), int(lay.stage_rows[l][s])
            d0, dn = int(lay.dev_off[s]), int(lay.dev_rows[s])
            segs.append([(hk[o:o + n], hv[o:o + n], int(lay.lo[l][s])),
                         (dk[d0:d0 + dn], dv[d0:d0 + dn], int(lay.h[s]))])
        return segs

    def free(self):
        self.k.free()
        self.v.free()
        self.dev_k = self.dev_v = None


class BatchedStack:
    """One arm (ring depth and budget) over a BatchedKV, one decode token at a time."""

    def __init__(self, torch, kvd, cfg, kv: BatchedKV, depth: int, budget_bytes: int, gemm_weights=None,
                 stream=None, pool: int = 4):
        self.torch, self.kvd, self.cfg, self.kv = torch, kvd, cfg, kv
        lay = self.layout = kv.layout
        self.depth = depth
        dev = torch.device("cuda:0")
        self.stream = stream or torch.cuda.Stream(device=dev)
        self.ring = kvd.Ring(depth, budget_bytes)
        rb = lay.row_bytes
        self.ordered_k = torch.empty(lay.cap_rows * rb, dtype=torch.uint8, device=dev)
        self.ordered_v = torch.empty(lay.cap_rows * rb, dtype=torch.uint8, device=dev)
        g = np.random.default_rng([cfg.seed, 7777])
        self.q = [torch.from_numpy(g.standard_normal((lay.n_seq, cfg.n_head_q, cfg.head_dim)).astype(np.float32)).to(dev)
                  for _ in range(lay.n_layers)]
        self.out = [torch.empty_like(self.q[0]) for _ in range(lay.n_layers)]
        self.ws = kvd.Workspace()
        self.gemm = gemm_weights
        if gemm_weights is not None:
            self.x = torch.randn(lay.n_seq, gemm_weights[0].shape[0], dtype=torch.bfloat16, device=dev,
                                 generator=torch.Generator(device=dev).manual_seed(cfg.seed))
            self.y = torch.empty(lay.n_seq, gemm_weights[0].shape[1], dtype=torch.bfloat16, device=dev)
        # newest rows written each step: a small seeded pool on the device
        from decode_attention_offloaded_amd import inputs
        gp = np.random.default_rng([cfg.seed, 4242])
        self.pool_k = [torch.from_numpy(inputs.random_kv_rows(gp, lay.n_seq, cfg.n_head_kv, cfg.head_dim)).to(dev)
                       for _ in range(pool)]
        self.pool_v = [torch.from_numpy(inputs.random_kv_rows(gp, lay.n_seq, cfg.n_head_kv, cfg.head_dim)).to(dev)
                       for _ in range(pool)]
        self.newest = torch.from_numpy(lay.dev_off + lay.dev_rows - 1).to(dev)
        self.q_pos = [int(x) for x in lay.q_pos]
        # segment tables: the device half never moves; the host half follows the view
        self._dev_segs = [[(int(kv.dev_k[l].data_ptr()) + int(lay.dev_off[s]) * rb,
                            int(kv.dev_v[l].data_ptr()) + int(lay.dev_off[s]) * rb,
                            int(lay.dev_rows[s]), int(lay.h[s]), rb) for s in range(lay.n_seq)]
                          for l in range(lay.n_layers)]

    def _stage(self, l, flags):
        lay = self.layout
        hk, hv = self.kv.host_ptrs(l)
        n = lay.stage_total[l]
        return self.ring.stage(l, flags, hk, hv, lay.row_bytes, n, n, lay.cap_rows, self.ordered_k.data_ptr(),
                               self.ordered_v.data_ptr(), stream=self.stream)

    def token(self, t: int):
        """One token over every layer; returns its time in ms (compute-stream events)."""
        torch, kvd, lay = self.torch, self.kvd, self.layout
        L, N, st = lay.n_layers, self.depth, self.stream
        rb = lay.row_bytes
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            e0.record(st)
            if N > 0:
                for l in range(min(N, L)):
                    if lay.stage_total[l]:
                        self._stage(l, kvd.STAGE_PREFETCH)
            for l in range(L):
                if self.gemm is not None:
                    torch.matmul(self.x, self.gemm[l % len(self.gemm)], out=self.y)
                p = (t * 7 + l) % len(self.pool_k)
                self.kv.dev_k[l].index_copy_(0, self.newest, self.pool_k[p])
                self.kv.dev_v[l].index_copy_(0, self.newest, self.pool_v[p])
                staged = lay.stage_total[l] > 0
                if staged:
                    _, view = self._stage(l, kvd.STAGE_ACQUIRE)
                    vk, vv, stride = view.k, view.v, view.row_stride
                else:
                    vk = vv = 0
                    stride = rb
                segs = []
                for s in range(lay.n_seq):
                    o, n = int(lay.stage_off[l][s]), int(lay.stage_rows[l][s])
                    host = (vk + o * stride, vv + o * stride, n, int(lay.lo[l][s]), stride) if n else (0, 0, 0, 0, rb)
                    segs.append([host, self._dev_segs[l][s]])
                kvd.attend_decode(self.q[l], self.out[l], segs, self.cfg.n_head_kv, window=lay.window[l],
                                  q_pos=self.q_pos, workspace=self.ws, stream=st)
                if staged:
                    self.ring.release(l, stream=st)
                if N > 0 and l + N < L and lay.stage_total[l + N]:
                    self._stage(l + N, kvd.STAGE_PREFETCH)
            e1.record(st)
        st.synchronize()
        return e0.elapsed_time(e1)

    def close(self):
        self.stream.synchronize()
        self.ring.close()
        self.ring = None


def run_batched(torch, kvd, inputs, cfg, lengths=None, n_layers=None, depths=(0, 1), budget_bytes=1 << 30,
                tokens=6, warmup=2, log=print, gemm=True, distinct_layers=None, window=None, check=None):
    """Ordered vs pipelined per-token time of the batched stack, arms A/B/B/A.

    check: optional callable(stack, layout, kv) run once on the last arm after
    its tokens (parity checks).  Returns a dict for the benchmark."""
    lengths = cfg4_lengths(cfg) if lengths is None else np.asarray(lengths)
    n_layers = n_layers or cfg.n_layers
    window = cfg.extra.get("window", 4096) if window is None else window
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    lay = BatchedLayout(lengths, n_layers, window, cfg.row_bytes)
    kv = BatchedKV(torch, inputs, cfg, lay, distinct=distinct_layers)
    log("batched KV: %d seqs (rows %d..%d, sum %d), %d layers, %.2f GB pinned, set up in %.1f s" %
        (lay.n_seq, int(lay.n.min()), int(lay.n.max()), int(lay.n.sum()), n_layers, 2 * lay.host_bytes / 1e9,
         time.perf_counter() - t0))
    weights = None
    if gemm:
        gen = torch.Generator(device=dev).manual_seed(cfg.seed)
        m, n = cfg.extra.get("gemv", (5120, 27648))
        weights = [(torch.randn(m, n, dtype=torch.bfloat16, device=dev, generator=gen) * 0.02)
                   for _ in range(n_layers)]
    order = list(depths) + list(reversed(depths))
    compute = torch.cuda.Stream(device=dev)
    times = {d: [] for d in depths}
    outs, stats, vram = {}, {}, {}
    for i, d in enumerate(order):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        free0 = torch.cuda.mem_get_info(dev)[0]
        st = BatchedStack(torch, kvd, cfg, kv, d, budget_bytes, gemm_weights=weights, stream=compute)
        for t in range(warmup):
            st.token(t)
        free1 = torch.cuda.mem_get_info(dev)[0]
        for t in range(warmup, warmup + tokens):
            times[d].append(st.token(t))
        outs[d] = [o.clone() for o in st.out]
        stats[d] = st.ring.stats()
        vram[d] = free0 - free1
        if check is not None and i == len(order) - 1:
            check(st, lay, kv)
        st.close()
        del st
        torch.cuda.empty_cache()
    identical = all(torch.equal(a, b) for a, b in zip(outs[depths[0]], outs[depths[-1]]))
    staged = lay.staged_bytes_per_token()
    res = {"n_seq": lay.n_seq, "lengths": [int(x) for x in lay.n], "n_layers": n_layers, "window": window,
           "tokens_timed": tokens, "order": order, "staged_bytes_per_token": staged,
           "visible_bytes_per_token": lay.visible_bytes_per_token(), "ring_cap_rows": lay.cap_rows,
           "bit_identical": bool(identical), "arms": {}}
    for d in depths:
        ms = float(np.median(times[d]))
        s = stats[d]
        res["arms"][str(d)] = {"depth": d, "ms_per_token": round(ms, 3), "tokens_per_s": round(1e3 / ms, 3),
                               "staged_GBps": round(staged / (ms * 1e-3) / 1e9, 2),
                               "ring_engaged_bytes": s["ring_bytes"] if s["engaged"] else 0,
                               "need_bytes": s["need_bytes"], "declined": s["declined"],
                               "vram_delta_bytes": int(vram[d]), "n_prefetch": s["n_prefetch"],
                               "n_acquire_pipelined": s["n_acquire_pipelined"],
                               "n_acquire_primed": s["n_acquire_primed"],
                               "n_acquire_ordered": s["n_acquire_ordered"], "bytes_early": s["bytes_early"],
                               "bytes_late": s["bytes_late"]}
    kv.free()
    del weights
    torch.cuda.empty_cache()
    return res
