"""Tile-streamed attention over a host-resident stack, through the staging ring.

Where a whole-layer ring does not fit the budget (a long context at a small
budget), each layer is attended in tiles of `tile_rows` rows instead: the
ring stages tiles, not layers, one attention call per tile leaves an
unnormalised partial result, and one merge per layer combines the tiles
("F5 — Advanced KV Cache Techniques", F5-opt W4, M7 Rolling KV: pinned-host
residency, a slot pool, a tile loop and an inter-tile online-softmax merge).
The ring and the kernels are the same as for whole layers: a tile is just a
delivery with its own key and a smaller capacity.

Per token and layer l: stand-in compute (bf16 GEMV); the host writes the
newest row (it falls in the last tile, so only that tile has a tail); for each
tile i: ACQUIRE delivery (l, i) -> partial attention over its rows -> RELEASE
-> PREFETCH the delivery N ahead (which may belong to layer l + 1); then the
merge of layer l's tiles into its output.  Deliveries are keyed l * T + i
and issued in that order, so the look-ahead crosses layer boundaries the way
it crosses tiles.
"""
from __future__ import annotations

import time

import numpy as np

from decode_attention_offloaded_amd.stack import HostKV, cfg_q, token_rows


class TiledStack:
    """One arm (ring depth and budget) of tile-streamed attention over a HostKV."""

    def __init__(self, torch, kvd, cfg, host: HostKV, n_rows: int, depth: int, budget_bytes: int,
                 tile_rows: int, gemv_weights=None, stream=None, new_rows=None):
        if tile_rows < 64 or tile_rows % 64:
            raise ValueError("tile_rows must be a positive multiple of 64")
        self.torch, self.kvd, self.cfg, self.host = torch, kvd, cfg, host
        self.n_rows, self.depth, self.tile_rows = n_rows, depth, tile_rows
        self.n_tiles = (n_rows + tile_rows - 1) // tile_rows
        dev = torch.device("cuda:0")
        self.stream = stream or torch.cuda.Stream(device=dev)
        self.ring = kvd.Ring(depth, budget_bytes)
        rb = host.row_bytes
        self.ordered_k = torch.empty(tile_rows * rb, dtype=torch.uint8, device=dev)
        self.ordered_v = torch.empty(tile_rows * rb, dtype=torch.uint8, device=dev)
        g = np.random.default_rng([cfg.seed, 7777])
        self.q = [torch.from_numpy(cfg_q(g, cfg)).to(dev) for _ in range(host.n_layers)]
        self.out = [torch.empty_like(self.q[0]) for _ in range(host.n_layers)]
        pf = kvd.partial_floats(1, cfg.n_head_q, cfg.head_dim)
        # one partial per tile, each starting on a 16-byte boundary
        self.pstride = (pf + 3) // 4 * 4
        if self.pstride != pf:
            raise ValueError("partial results must pack back to back")
        self.partials = torch.empty(self.n_tiles * pf, dtype=torch.float32, device=dev)
        self.ws = kvd.Workspace()
        self.gemv = gemv_weights
        if gemv_weights is not None:
            self.x = torch.randn(1, gemv_weights[0].shape[0], dtype=torch.bfloat16, device=dev,
                                 generator=torch.Generator(device=dev).manual_seed(cfg.seed))
            self.y = torch.empty(1, gemv_weights[0].shape[1], dtype=torch.bfloat16, device=dev)
        self.new_rows = new_rows

    def _tile(self, i):
        r0 = i * self.tile_rows
        return r0, min(self.tile_rows, self.n_rows - r0)

    def _stage(self, d, flags):
        h, T = self.host, self.n_tiles
        layer, i = divmod(d, T)
        r0, n = self._tile(i)
        # the newest row (n_rows - 1) is written each step: it sits in the last tile
        stable = n - 1 if r0 + n == self.n_rows else n
        off = r0 * h.row_bytes
        return self.ring.stage(d, flags, h.k_ptr(layer) + off, h.v_ptr(layer) + off, h.row_bytes, n, stable,
                               self.tile_rows, self.ordered_k.data_ptr(), self.ordered_v.data_ptr(),
                               stream=self.stream)

    def token(self, t: int):
        """One decode token over every layer; returns its time in ms (compute-stream events)."""
        torch, kvd, h = self.torch, self.kvd, self.host
        L, T, N, s = h.n_layers, self.n_tiles, self.depth, self.stream
        total = L * T
        pf = self.pstride
        qpos = [self.n_rows - 1]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            for d in range(min(N, total)):
                self._stage(d, kvd.STAGE_PREFETCH)
            for l in range(L):
                if self.gemv is not None:
                    torch.matmul(self.x, self.gemv[l % len(self.gemv)], out=self.y)
                if self.new_rows is not None:
                    kr, vr = self.new_rows(t, l)
                    h.k_rows(l)[self.n_rows - 1] = kr
                    h.v_rows(l)[self.n_rows - 1] = vr
                for i in range(T):
                    d = l * T + i
                    r0, n = self._tile(i)
                    _, view = self._stage(d, kvd.STAGE_ACQUIRE)
                    kvd.attend_decode_partial(self.q[l], self.partials[i * pf:(i + 1) * pf],
                                              [[(view.k, view.v, n, r0, view.row_stride)]], self.cfg.n_head_kv,
                                              q_pos=qpos, workspace=self.ws, stream=s)
                    self.ring.release(d, stream=s)
                    if N > 0 and d + N < total:
                        self._stage(d + N, kvd.STAGE_PREFETCH)
                kvd.attend_merge(self.partials, T, self.out[l], stream=s)
            e1.record(s)
        s.synchronize()
        return e0.elapsed_time(e1)

    def close(self):
        self.stream.synchronize()
        self.ring.close()
        self.ring = None


def run_tiled(torch, kvd, inputs, cfg, n_layers=64, depths=(0, 1), budget_bytes=128 << 20, tile_rows=None,
              tokens=3, warmup=1, log=print, n_rows=None, gemv=True, distinct_layers=None, host=None):
    """Ordered vs pipelined per-token time of tile-streamed attention, arms
    A/B/B/A; tile_rows defaults to the largest tile a depth-max(depths) ring of
    this budget holds.  Returns a dict for the benchmark."""
    n_rows = n_rows or cfg.n_ctx
    dev = torch.device("cuda:0")
    if tile_rows is None:
        rc, tile_rows = kvd.tile_rows(max(max(depths), 1), budget_bytes, cfg.row_bytes)
        if rc != kvd.KVD_OK:
            raise ValueError("no tile fits a ring of %d bytes" % budget_bytes)
    own_host = host is None
    t0 = time.perf_counter()
    if own_host:
        host = HostKV(n_layers, n_rows, cfg.row_bytes)
        host.fill(inputs, cfg, n_rows, distinct=distinct_layers)
        log("host KV: %d layers x %d rows, %.2f GB pinned, filled in %.1f s" %
            (n_layers, n_rows, 2 * host.k.nbytes / 1e9, time.perf_counter() - t0))
    weights = None
    if gemv:
        gen = torch.Generator(device=dev).manual_seed(cfg.seed)
        m, n = cfg.extra.get("gemv", (5120, 27648))
        weights = [(torch.randn(m, n, dtype=torch.bfloat16, device=dev, generator=gen) * 0.02)
                   for _ in range(n_layers)]
    rows_fn = token_rows(cfg)
    order = list(depths) + list(reversed(depths))
    compute = torch.cuda.Stream(device=dev)
    times = {d: [] for d in depths}
    outs, stats, vram = {}, {}, {}
    for d in order:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        free0 = torch.cuda.mem_get_info(dev)[0]
        st = TiledStack(torch, kvd, cfg, host, n_rows, d, budget_bytes, tile_rows, gemv_weights=weights,
                        new_rows=rows_fn, stream=compute)
        for t in range(warmup):
            st.token(t)
        free1 = torch.cuda.mem_get_info(dev)[0]
        for t in range(warmup, warmup + tokens):
            times[d].append(st.token(t))
        outs[d] = [o.clone() for o in st.out]
        stats[d] = st.ring.stats()
        vram[d] = free0 - free1
        n_tiles = st.n_tiles
        st.close()
        del st
        torch.cuda.empty_cache()
    identical = all(torch.equal(a, b) for a, b in zip(outs[depths[0]], outs[depths[-1]]))
    bytes_token = 2 * n_layers * n_rows * cfg.row_bytes
    res = {"n_ctx": n_rows, "n_layers": n_layers, "tile_rows": tile_rows, "tiles_per_layer": n_tiles,
           "budget_bytes": budget_bytes, "tokens_timed": tokens, "order": order, "bytes_per_token": bytes_token,
           "bit_identical": bool(identical), "arms": {}}
    for d in depths:
        ms = float(np.median(times[d]))
        s = stats[d]
        res["arms"][str(d)] = {"depth": d, "ms_per_token": round(ms, 3), "tokens_per_s": round(1e3 / ms, 3),
                               "staged_GBps": round(bytes_token / (ms * 1e-3) / 1e9, 2),
                               "ring_engaged_bytes": s["ring_bytes"] if s["engaged"] else 0,
                               "need_bytes": s["need_bytes"], "declined": s["declined"],
                               "vram_delta_bytes": int(vram[d]), "n_prefetch": s["n_prefetch"],
                               "n_acquire_pipelined": s["n_acquire_pipelined"],
                               "n_acquire_primed": s["n_acquire_primed"],
                               "n_acquire_ordered": s["n_acquire_ordered"], "bytes_early": s["bytes_early"],
                               "bytes_late": s["bytes_late"]}
    res["outs"] = outs[depths[-1]]
    if own_host:
        host.free()
    del weights
    torch.cuda.empty_cache()
    return res
