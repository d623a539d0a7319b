"""The staging ring's logic on the CPU: the product's ring core compiled with a
simulated device runtime (tests/ringsim).  Simulated streams execute in
random interleavings; CHECK operations on the compute stream (where attention
would read the slot) compare device bytes with what the host rows held when
the layer was acquired.  Fresh device memory is 0xFF so undelivered bytes show.

What is checked follows "sched: pipeline the delivery of a host-resident KV
cache (R4)": What it does 1-3 (stable prefix, ring with a ready/release pair
per slot, N + 2 slots and stream-to-stream recycling), the depth knob, and
Device memory (budget before allocation, latched, lazy transport)."""
import ctypes

import numpy as np
import pytest

from decode_attention_offloaded_amd import kvd

MiB = 1 << 20


@pytest.fixture(scope="module")
def sim_lib():
    from tests import ringsim_build
    L = ctypes.CDLL(ringsim_build.build())
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.sim_new.restype = vp
    L.sim_new.argtypes = [ctypes.c_uint64]
    L.sim_delete.argtypes = [vp]
    L.sim_configure.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64]
    L.sim_stream_new.restype = vp
    L.sim_stream_new.argtypes = [vp]
    L.sim_ring_create.restype = vp
    L.sim_ring_create.argtypes = [vp, ctypes.c_int32, i64]
    L.sim_check.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, i64]
    L.sim_run.restype = ctypes.c_int
    L.sim_run.argtypes = [vp, ctypes.c_int]
    L.sim_drain.restype = ctypes.c_int
    L.sim_drain.argtypes = [vp]
    L.sim_counter.restype = i64
    L.sim_counter.argtypes = [vp, ctypes.c_int]
    L.sim_executed.restype = i64
    L.sim_executed.argtypes = [vp, ctypes.c_int]
    L.sim_log.restype = ctypes.c_char_p
    L.sim_log.argtypes = [vp]
    L.kvd_ring_stage_layer.restype = ctypes.c_int
    L.kvd_ring_stage_layer.argtypes = [vp, ctypes.POINTER(kvd.StageArgs), vp, ctypes.POINTER(kvd.SlotView)]
    L.kvd_ring_release.restype = ctypes.c_int
    L.kvd_ring_release.argtypes = [vp, ctypes.c_int32, vp]
    L.kvd_ring_stats_get.restype = ctypes.c_int
    L.kvd_ring_stats_get.argtypes = [vp, ctypes.POINTER(kvd.RingStats), ctypes.c_size_t]
    L.kvd_ring_destroy.argtypes = [vp]
    L.kvd_last_error.restype = ctypes.c_char_p
    return L


ERRORS, DEV_BYTES, PEAK, LIVE, DEADLOCKS, SYNCS, STREAMS, QUEUED = range(8)
COPY, RECORD, WAIT, CHECK = range(4)


class Harness:
    """A host-resident stack of layers driven through a simulated ring."""

    def __init__(self, L, depth, budget, n_layers, cap_rows, row_bytes=64, seed=0, fail_after=-1, v_row_bytes=0):
        self.L = L
        self.sim = L.sim_new(seed)
        L.sim_configure(self.sim, 1, 0, fail_after)
        self.compute = L.sim_stream_new(self.sim)
        self.ring = L.sim_ring_create(self.sim, depth, budget)
        self.depth, self.n_layers, self.cap, self.rb = depth, n_layers, cap_rows, row_bytes
        self.vrb_arg = v_row_bytes
        self.vrb = v_row_bytes or row_bytes
        self.rng = np.random.default_rng(seed)
        self.hk = self.rng.integers(0, 256, (n_layers, cap_rows, row_bytes), dtype=np.uint8)
        self.hv = self.rng.integers(0, 256, (n_layers, cap_rows, self.vrb), dtype=np.uint8)
        self.ok = np.zeros(cap_rows * row_bytes, np.uint8)   # "device" ordered buffers (simulated memory is host memory)
        self.ov = np.zeros(cap_rows * self.vrb, np.uint8)
        self.n_checks = 0

    def args(self, layer, flags, n_rows, stable=None, cap=None, rb=None):
        rb = rb or self.rb
        return kvd.StageArgs(layer, flags, self.hk[layer].ctypes.data, self.hv[layer].ctypes.data, rb, n_rows,
                             n_rows - 1 if stable is None else stable, cap or self.cap, self.ok.ctypes.data,
                             self.ov.ctypes.data, self.vrb_arg)

    def stage(self, layer, flags, n_rows, **kw):
        a = self.args(layer, flags, n_rows, **kw)
        view = kvd.SlotView()
        rc = self.L.kvd_ring_stage_layer(self.ring, ctypes.byref(a), self.compute, ctypes.byref(view))
        return rc, view

    def check(self, layer, view, n_rows):
        self.L.sim_check(self.sim, self.compute, view.k, self.hk[layer].ctypes.data, n_rows * self.rb, self.n_checks)
        self.L.sim_check(self.sim, self.compute, view.v, self.hv[layer].ctypes.data, n_rows * self.vrb,
                         self.n_checks + 1)
        self.n_checks += 2

    def step(self, hi=6):
        self.L.sim_run(self.sim, int(self.rng.integers(0, hi)))

    def token(self, n_rows, run_hi=6):
        """Prefetch the first N layers, then per layer: new row, ACQUIRE, check, RELEASE, PREFETCH l+N."""
        N, L = self.depth, self.L
        for l in range(min(N, self.n_layers)):
            rc, _ = self.stage(l, kvd.STAGE_PREFETCH, n_rows)
            assert rc in (kvd.KVD_OK, kvd.KVD_DECLINED), self.err()
            self.step(run_hi)
        for l in range(self.n_layers):
            self.hk[l, n_rows - 1] = self.rng.integers(0, 256, self.rb, dtype=np.uint8)
            self.hv[l, n_rows - 1] = self.rng.integers(0, 256, self.vrb, dtype=np.uint8)
            rc, view = self.stage(l, kvd.STAGE_ACQUIRE, n_rows)
            assert rc in (kvd.KVD_OK, kvd.KVD_DECLINED), self.err()
            self.check(l, view, n_rows)
            self.step(run_hi)
            assert L.kvd_ring_release(self.ring, l, self.compute) == kvd.KVD_OK, self.err()
            if N > 0 and l + N < self.n_layers:
                rc, _ = self.stage(l + N, kvd.STAGE_PREFETCH, n_rows)
                assert rc in (kvd.KVD_OK, kvd.KVD_DECLINED), self.err()
            self.step(run_hi)
        assert L.sim_drain(self.sim) == 0, self.log()   # the step's final synchronisation

    def stats(self):
        st = kvd.RingStats()
        assert self.L.kvd_ring_stats_get(self.ring, ctypes.byref(st), ctypes.sizeof(st)) == 0
        return {n: getattr(st, n) for n, _ in kvd.RingStats._fields_}

    def counter(self, which):
        return self.L.sim_counter(self.sim, which)

    def err(self):
        return self.L.kvd_last_error().decode()

    def log(self):
        return self.L.sim_log(self.sim).decode()

    def close(self):
        if self.ring:
            self.L.kvd_ring_destroy(self.ring)
            self.ring = None
        assert self.counter(LIVE) == 0, "device memory leaked"
        self.L.sim_delete(self.sim)


@pytest.mark.parametrize("depth", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n_layers", [1, 5, 7, 64])
@pytest.mark.parametrize("seed", [0, 1])
def test_random_interleavings_deliver_exact_bytes(sim_lib, depth, n_layers, seed):
    h = Harness(sim_lib, depth, 1 << 40, n_layers, 40, seed=seed)
    for t in range(3):
        h.token(40 - t)   # the context shrinks a row per step here; capacity stays
    assert h.counter(ERRORS) == 0, h.log()
    assert h.counter(DEADLOCKS) == 0
    st = h.stats()
    assert st["n_acquire_ordered"] == 0
    assert st["n_acquire_pipelined"] + st["n_acquire_primed"] == 3 * n_layers
    assert st["n_acquire_primed"] == 0   # the first N layers are prefetched at the token start
    assert h.counter(SYNCS) == 0         # never synchronises through the host
    h.close()


def test_checker_catches_stale_prefix(sim_lib):
    """Negative control: a caller that rewrites prefix rows after they were
    delivered (breaking the stable-prefix contract) is caught by the checks."""
    h = Harness(sim_lib, 1, 1 << 40, 3, 16, seed=3)
    rc, _ = h.stage(0, kvd.STAGE_PREFETCH, 16)
    assert rc == kvd.KVD_OK
    assert sim_lib.sim_drain(h.sim) == 0
    h.hk[0, 3] ^= 0xFF
    rc, view = h.stage(0, kvd.STAGE_ACQUIRE, 16)
    h.check(0, view, 16)
    assert sim_lib.sim_drain(h.sim) == 0
    assert h.counter(ERRORS) >= 1
    assert sim_lib.kvd_ring_release(h.ring, 0, h.compute) == 0
    h.close()


def test_look_ahead_deeper_than_the_ring_is_refused(sim_lib):
    """N + 2 slots: a fourth delivery before any release would reuse a slot still
    in use -- the ring refuses instead of racing."""
    h = Harness(sim_lib, 1, 1 << 40, 8, 16)
    for l in range(3):
        rc, _ = h.stage(l, kvd.STAGE_PREFETCH, 16)
        assert rc == kvd.KVD_OK
    rc, _ = h.stage(3, kvd.STAGE_PREFETCH, 16)
    assert rc == kvd.KVD_ESTATE and "release" in h.err()
    rc, _ = h.stage(1, kvd.STAGE_PREFETCH, 16)
    assert rc == kvd.KVD_ESTATE   # staged twice
    for l in range(3):
        rc, view = h.stage(l, kvd.STAGE_ACQUIRE, 16)
        assert rc == kvd.KVD_OK
        h.check(l, view, 16)
        assert sim_lib.kvd_ring_release(h.ring, l, h.compute) == 0
    assert sim_lib.kvd_ring_release(h.ring, 2, h.compute) == kvd.KVD_ESTATE   # not acquired any more
    assert sim_lib.sim_drain(h.sim) == 0 and h.counter(ERRORS) == 0
    h.close()


def test_slot_cursor_does_not_alias_across_steps(sim_lib):
    """64 layers on 3 slots: layer 63 and the next step's layer 0 take
    different slots (a monotonic cursor, not layer mod slots)."""
    h = Harness(sim_lib, 1, 1 << 40, 64, 8, seed=4)
    slots = []
    for t in range(2):
        for l in range(1):
            h.stage(l, kvd.STAGE_PREFETCH, 8)
        for l in range(64):
            rc, view = h.stage(l, kvd.STAGE_ACQUIRE, 8)
            slots.append(view.slot)
            h.check(l, view, 8)
            sim_lib.kvd_ring_release(h.ring, l, h.compute)
            if l + 1 < 64:
                h.stage(l + 1, kvd.STAGE_PREFETCH, 8)
        assert sim_lib.sim_drain(h.sim) == 0
    assert slots == [i % 3 for i in range(128)]
    assert h.counter(ERRORS) == 0
    h.close()


def test_tail_placement(sim_lib):
    """At every depth the tail (K and V) is copied on the compute stream, so the
    transfer streams carry only prefix copies: 2 tail copies per prefetched
    layer on the compute stream, and nothing else there."""
    for depth in (1, 2):
        h = Harness(sim_lib, depth, 1 << 40, 6, 16, seed=5)
        h.token(16)
        assert sim_lib.sim_executed(h.compute, COPY) == 2 * 6, depth
        assert h.counter(ERRORS) == 0
        h.close()


def test_stats_account_for_every_byte(sim_lib):
    rb, n, L = 64, 20, 6
    h = Harness(sim_lib, 1, 1 << 40, L, n, row_bytes=rb)
    h.token(n)
    st = h.stats()
    assert st["n_prefetch"] == L
    assert st["bytes_early"] == L * 2 * (n - 1) * rb
    assert st["bytes_late"] == L * 2 * rb
    assert st["ring_bytes"] == 3 * 2 * n * rb and st["engaged"] == 1
    h.close()


# ------------------------------------------------------------------ budget and lifetime

def test_depth_zero_is_the_ordered_path_and_creates_nothing(sim_lib):
    h = Harness(sim_lib, 0, 1 << 40, 5, 16)
    h.token(16)
    st = h.stats()
    assert st["n_acquire_ordered"] == 5 and st["engaged"] == 0 and st["declined"] == 0
    assert h.counter(STREAMS) == 0 and h.counter(PEAK) == 0
    assert h.counter(ERRORS) == 0
    h.close()


def test_lazy_transport(sim_lib):
    h = Harness(sim_lib, 2, 1 << 40, 5, 16)
    assert h.counter(STREAMS) == 0 and h.counter(PEAK) == 0
    h.token(16)
    assert h.counter(STREAMS) == 2   # K and V transfer streams
    h.close()


def test_over_budget_declines_before_allocating(sim_lib):
    need = 3 * 2 * 16 * 64
    h = Harness(sim_lib, 1, need - 1, 5, 16)
    h.token(16)
    st = h.stats()
    assert st["declined"] == 1 and st["engaged"] == 0 and st["need_bytes"] == need
    assert st["n_acquire_ordered"] == 5
    assert h.counter(PEAK) == 0 and h.counter(STREAMS) == 0
    assert h.counter(ERRORS) == 0
    h.close()
    h = Harness(sim_lib, 1, need, 5, 16)   # inclusive: exactly the budget fits
    h.token(16)
    assert h.stats()["engaged"] == 1 and h.counter(PEAK) == need
    h.close()


def test_decline_is_latched(sim_lib):
    rb = 64
    h = Harness(sim_lib, 1, 3 * 2 * 32 * rb, 4, 64, row_bytes=rb)
    h.token(32)  # plan with cap 64 would not fit ... but the harness passes cap=64
    st = h.stats()
    assert st["declined"] == 1
    # shrinking the capacity later does not re-engage: declines are latched
    rc, view = h.stage(0, kvd.STAGE_ACQUIRE, 16, cap=16)
    assert rc == kvd.KVD_DECLINED and view.pipelined == 0
    assert h.counter(PEAK) == 0
    sim_lib.sim_drain(h.sim)
    h.close()


def test_growth_past_budget_tears_down_then_stays_declined(sim_lib):
    rb = 64
    budget = 3 * 2 * 32 * rb
    h = Harness(sim_lib, 1, budget, 4, 64, row_bytes=rb)
    rc, _ = h.stage(0, kvd.STAGE_ACQUIRE, 16, cap=32)
    assert rc == kvd.KVD_OK and h.counter(DEV_BYTES) == budget
    assert sim_lib.kvd_ring_release(h.ring, 0, h.compute) == 0
    # capacity grows while a delivery is in flight: refused, not raced
    rc, _ = h.stage(1, kvd.STAGE_PREFETCH, 16, cap=32)
    assert rc == kvd.KVD_OK
    rc, _ = h.stage(2, kvd.STAGE_ACQUIRE, 16, cap=64)
    assert rc == kvd.KVD_ESTATE
    rc, view = h.stage(1, kvd.STAGE_ACQUIRE, 16, cap=32)
    assert rc == kvd.KVD_OK
    assert sim_lib.kvd_ring_release(h.ring, 1, h.compute) == 0
    # quiescent: the over-budget plan frees the ring and latches the decline
    rc, view = h.stage(2, kvd.STAGE_ACQUIRE, 16, cap=64)
    assert rc == kvd.KVD_DECLINED and view.pipelined == 0
    assert h.counter(DEV_BYTES) == 0
    st = h.stats()
    assert st["declined"] == 1 and st["engaged"] == 0
    assert sim_lib.sim_drain(h.sim) == 0 and h.counter(ERRORS) == 0
    h.close()


def test_growth_within_budget_reallocates_when_quiescent(sim_lib):
    rb = 64
    h = Harness(sim_lib, 1, 1 << 40, 4, 64, row_bytes=rb)
    rc, _ = h.stage(0, kvd.STAGE_ACQUIRE, 16, cap=32)
    assert rc == kvd.KVD_OK and h.counter(DEV_BYTES) == 3 * 2 * 32 * rb
    sim_lib.kvd_ring_release(h.ring, 0, h.compute)
    rc, view = h.stage(1, kvd.STAGE_ACQUIRE, 16, cap=64)
    assert rc == kvd.KVD_OK and h.counter(DEV_BYTES) == 3 * 2 * 64 * rb
    h.check(1, view, 16)
    sim_lib.kvd_ring_release(h.ring, 1, h.compute)
    assert sim_lib.sim_drain(h.sim) == 0 and h.counter(ERRORS) == 0
    h.close()


@pytest.mark.parametrize("fail_after", [0, 1, 3, 5])
def test_allocation_failure_declines_without_leaking(sim_lib, fail_after):
    h = Harness(sim_lib, 1, 1 << 40, 3, 16, fail_after=fail_after)
    h.token(16)
    st = h.stats()
    assert st["declined"] == 1 and st["engaged"] == 0 and st["n_acquire_ordered"] == 3
    assert h.counter(LIVE) == 0 and h.counter(DEV_BYTES) == 0
    assert h.counter(ERRORS) == 0
    h.close()


def test_pageable_and_wrong_device_are_refused(sim_lib):
    h = Harness(sim_lib, 1, 1 << 40, 3, 16)
    sim_lib.sim_configure(h.sim, 0, 0, -1)
    rc, _ = h.stage(0, kvd.STAGE_ACQUIRE, 16)
    assert rc == kvd.KVD_EINVAL and "pinned" in h.err()
    sim_lib.sim_configure(h.sim, 1, 0, -1)
    rc, _ = h.stage(0, kvd.STAGE_ACQUIRE, 16)
    assert rc == kvd.KVD_OK
    sim_lib.sim_configure(h.sim, 1, 1, -1)
    rc, _ = h.stage(1, kvd.STAGE_ACQUIRE, 16)
    assert rc == kvd.KVD_ESTATE and "device" in h.err()
    sim_lib.sim_configure(h.sim, 1, 0, -1)
    assert sim_lib.kvd_ring_release(h.ring, 0, h.compute) == 0
    assert sim_lib.sim_drain(h.sim) == 0
    h.close()


def test_planner_matches_the_oracle(sim_lib, oracle):
    """The product planner's size and decision equal the oracle's (which is
    pinned to the page's printed ring column) over a sweep."""
    rng = np.random.default_rng(11)
    for _ in range(60):
        depth = int(rng.integers(0, 5))
        cap = int(rng.integers(1, 64))
        rb = int(rng.integers(1, 16)) * 64
        budget = int(rng.integers(0, (depth + 2) * 2 * cap * rb * 2 + 1))
        h = Harness(sim_lib, depth, budget, 2, cap, row_bytes=rb)
        rc, view = h.stage(0, kvd.STAGE_ACQUIRE, cap)
        st = h.stats()
        fits = oracle.ring_fits(depth, cap, rb, budget)
        assert (rc == kvd.KVD_OK) == fits
        if depth > 0:
            assert st["need_bytes"] == oracle.ring_bytes(depth, cap, rb)
        sim_lib.kvd_ring_release(h.ring, 0, h.compute)
        sim_lib.sim_drain(h.sim)
        h.close()


@pytest.mark.parametrize("depth", [1, 2, 4])
@pytest.mark.parametrize("seed", range(4))
def test_narrow_v_rows_stage_exactly(sim_lib, depth, seed):
    """V rows shorter than K rows (a q4_0 V cache): every view holds the host
    K and V bytes, under random interleavings; the ring is sized
    (N + 2) x cap x (K row + V row) and the counters count both."""
    rb, vrb, n, layers = 64, 36, 40, 6
    need = (depth + 2) * n * (rb + vrb)
    h = Harness(sim_lib, depth, need, layers, n, row_bytes=rb, seed=seed, v_row_bytes=vrb)
    for _ in range(3):
        h.token(n)
    st = h.stats()
    assert st["engaged"] == 1 and st["need_bytes"] == need and st["ring_bytes"] == need
    assert st["n_acquire_ordered"] == 0
    assert st["bytes_early"] + st["bytes_late"] == 3 * layers * n * (rb + vrb)
    # one byte less of budget declines, before anything is allocated
    h2 = Harness(sim_lib, depth, need - 1, layers, n, row_bytes=rb, seed=seed, v_row_bytes=vrb)
    h2.token(n)
    st2 = h2.stats()
    assert st2["declined"] == 1 and st2["n_acquire_ordered"] == layers and st2["bytes_ordered"] == layers * n * (rb + vrb)
