"""GPU tests of the staging ring through the C ABI: the pipelined path must be
bit-identical to the ordered path (byte-identical output at depths 0/1/4/8 is
the validation "sched: pipeline the delivery of a host-resident KV cache (R4)"
uses), the budget must decline before allocating, and no ordering slip may
show under consumer delays and slot poisoning."""
import ctypes

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

pytestmark = pytest.mark.gpu
MiB = 1 << 20


@pytest.fixture(scope="module")
def env():
    import torch
    from decode_attention_offloaded_amd import kvd, stack
    return torch, kvd, stack


def small_cfg():
    return inputs.Config(90, "ring_test", 12, 1, 3000, 40, 8, 128)


def run_arm(env, cfg, host, n_rows, depth, budget, tokens, hook=None, after=None, xfer_delay_us=0, seed=1):
    torch, kvd, stack = env
    st = stack.Stack(torch, kvd, cfg, host, n_rows, depth, budget, new_rows=stack.token_rows(cfg))
    st.on_view = hook
    st.after_attend = after
    if xfer_delay_us:
        st.ring.set_transfer_delay(xfer_delay_us, seed)
    outs = []
    for t in range(tokens):
        st.token(t)
        # cloned on the stack's stream: the next token's attention writes
        # `out` on that stream, so a clone on another stream could race it
        with torch.cuda.stream(st.stream):
            outs.append([o.clone() for o in st.out])
    s = st.ring.stats()
    st.close()
    return outs, s


def test_pipelined_is_bit_identical_to_ordered(env, oracle):
    torch, kvd, stack = env
    cfg = small_cfg()
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    ref, s0 = run_arm(env, cfg, host, cfg.n_ctx, 0, 0, 3)
    assert s0["engaged"] == 0 and s0["n_acquire_ordered"] == 3 * cfg.n_layers
    for depth in (1, 2, 4, 8):
        outs, s = run_arm(env, cfg, host, cfg.n_ctx, depth, 1 << 30, 3)
        assert s["n_acquire_ordered"] == 0 and s["n_acquire_pipelined"] == 3 * cfg.n_layers, s
        for t in range(3):
            for l in range(cfg.n_layers):
                assert torch.equal(outs[t][l], ref[t][l]), (depth, t, l)
    # and the last token agrees with the oracle on two layers
    st = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, 0, 0)
    for l in (0, cfg.n_layers - 1):
        q = st.q[l].cpu().numpy()
        k = host.k_rows(l)[:cfg.n_ctx].copy()
        v = host.v_rows(l)[:cfg.n_ctx].copy()
        r = oracle.attend(q, [[(k, v, 0)]], cfg.n_head_kv, cfg.head_dim, threads=8)
        assert np.max(np.abs(ref[-1][l].cpu().numpy() - r)) <= 1e-3
    st.close()
    host.free()


def test_consumer_delays_and_poisoned_slots(env):
    """Slow consumer (spin kernel before every attention) and every slot
    overwritten with 0xFF (a NaN binary16 scale) right after its attention and
    before its release: a delivery that did not wait for the release, or an
    attention that did not wait for its delivery, would read poison."""
    torch, kvd, stack = env
    cfg = small_cfg()
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    ref, _ = run_arm(env, cfg, host, cfg.n_ctx, 0, 0, 2)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemsetAsync.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]
    rng = np.random.default_rng(5)

    def delay(layer, view):
        torch.cuda._sleep(int(rng.integers(1000, 200000)))

    def poison(layer, view):
        if view.pipelined:
            s = torch.cuda.current_stream().cuda_stream
            n = host.cap_rows * host.row_bytes
            assert hip.hipMemsetAsync(view.k, 0xFF, n, s) == 0
            assert hip.hipMemsetAsync(view.v, 0xFF, n, s) == 0

    for depth in (1, 2, 4):
        outs, s = run_arm(env, cfg, host, cfg.n_ctx, depth, 1 << 30, 2, hook=delay, after=poison)
        assert s["n_acquire_pipelined"] == 2 * cfg.n_layers
        for t in range(2):
            for l in range(cfg.n_layers):
                assert torch.isfinite(outs[t][l]).all(), (depth, t, l)
                assert torch.equal(outs[t][l], ref[t][l]), (depth, t, l)
    host.free()


def test_transfer_delays_and_poisoned_slots(env):
    """Slow deliveries: before every copy on the ring's transfer streams the
    stream is held for a random 0..5 ms (a spin kernel on that stream, longer
    than the host takes to enqueue a layer), so prefix and tail copies land
    after the attention that needs them was enqueued, while every slot is
    overwritten with 0xFF after its attention and before its release.  An attention that did not wait for its delivery would
    read the previous layer's bytes or the poison; a delivery that did not wait
    for the release would be poisoned."""
    torch, kvd, stack = env
    cfg = small_cfg()
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    ref, _ = run_arm(env, cfg, host, cfg.n_ctx, 0, 0, 2)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemsetAsync.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]

    def poison(layer, view):
        if view.pipelined:
            s = torch.cuda.current_stream().cuda_stream
            n = host.cap_rows * host.row_bytes
            assert hip.hipMemsetAsync(view.k, 0xFF, n, s) == 0
            assert hip.hipMemsetAsync(view.v, 0xFF, n, s) == 0

    import time
    wall = {}
    run_arm(env, cfg, host, cfg.n_ctx, 1, 1 << 30, 2)   # warm-up, not timed
    for depth, seed, delay in ((1, 10, 0), (1, 11, 5000), (2, 12, 5000), (4, 13, 5000)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        outs, s = run_arm(env, cfg, host, cfg.n_ctx, depth, 1 << 30, 2, after=poison, xfer_delay_us=delay, seed=seed)
        torch.cuda.synchronize()
        wall[(depth, delay)] = time.perf_counter() - t0
        assert s["n_acquire_pipelined"] == 2 * cfg.n_layers
        for t in range(2):
            for l in range(cfg.n_layers):
                assert torch.isfinite(outs[t][l]).all(), (depth, t, l)
                assert torch.equal(outs[t][l], ref[t][l]), (depth, t, l)
    # the holds are real: at depth 1 each of the 24 deliveries waits 2.5 ms on
    # average per stream, so the two tokens take tens of milliseconds longer
    print("wall time of two tokens (s):", wall)
    assert wall[(1, 5000)] > wall[(1, 0)] + 0.02, wall
    host.free()


@pytest.mark.parametrize("depth,budget_mib,fits", [(1, 128, False), (1, 1024, True), (2, 128, False),
                                                   (2, 1024, False), (0, 1024, False)])
def test_decline_matrix_long_context(env, depth, budget_mib, fits):
    """131072-row capacity: depth 1 needs 816 MiB (fits 1 GiB, not 128 MiB);
    depth 2 needs 1088 MiB (fits neither).  A declined ring allocates nothing
    and the output equals the ordered path."""
    torch, kvd, stack = env
    cfg = inputs.Config(91, "decline", 3, 1, 131072, 40, 8, 128)
    n_rows = 512
    host = stack.HostKV(cfg.n_layers, n_rows, cfg.row_bytes)
    host.fill(inputs, cfg, n_rows)
    torch.cuda.synchronize()
    ring = kvd.Ring(depth, budget_mib * MiB)
    dev = torch.device("cuda:0")
    ok = torch.empty(n_rows * cfg.row_bytes, dtype=torch.uint8, device=dev)
    ov = torch.empty_like(ok)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(dev)[0]
    rc, view = ring.stage(0, kvd.STAGE_ACQUIRE, host.k_ptr(0), host.v_ptr(0), cfg.row_bytes, n_rows, n_rows - 1,
                          cfg.n_ctx, ok.data_ptr(), ov.data_ptr())
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(dev)[0]
    st = ring.stats()
    if fits:
        assert rc == kvd.KVD_OK and view.pipelined == 1 and st["engaged"] == 1
        assert st["ring_bytes"] == 3 * 2 * 131072 * cfg.row_bytes
        # device free memory is reported at a coarse granularity: allow 4 MiB
        assert st["ring_bytes"] - 4 * MiB <= free0 - free1 <= budget_mib * MiB
    else:
        assert rc == kvd.KVD_DECLINED and view.pipelined == 0
        assert st["engaged"] == 0 and st["ring_bytes"] == 0
        assert free0 - free1 < 4 * MiB
        if depth > 0:
            assert st["declined"] == 1
            assert st["need_bytes"] == (depth + 2) * 2 * 131072 * cfg.row_bytes
    ring.release(0)
    ring.close()
    host.free()


def test_vram_growth_is_the_ring(env):
    torch, kvd, stack = env
    cfg = inputs.Config(92, "vram", 6, 1, 16384, 40, 8, 128)
    res = stack.run_host_resident(torch, kvd, inputs, cfg, n_layers=6, depths=(0, 1), budget_bytes=128 * MiB,
                                  tokens=2, warmup=1, log=lambda *a: None, gemv=False)
    a0, a1 = res["arms"]["0"], res["arms"]["1"]
    assert res["bit_identical"]
    ring = a1["ring_engaged_bytes"]
    assert ring == 3 * 2 * 16384 * cfg.row_bytes <= 128 * MiB
    grow = a1["vram_delta_bytes"] - a0["vram_delta_bytes"]
    assert ring - 4 * MiB <= grow <= ring + 8 * MiB, (grow, ring)


def test_ordered_path_never_creates_the_transport(env):
    torch, kvd, stack = env
    ring = kvd.Ring(0, 1 << 30)
    st = ring.stats()
    assert st["engaged"] == 0 and st["ring_bytes"] == 0 and st["n_slots"] == 0
    ring.close()
    r1 = kvd.Ring(1, 1 << 30)
    assert r1.stats()["engaged"] == 0  # lazy: nothing before the first stage
    r1.close()


def test_pageable_host_memory_is_rejected(env):
    torch, kvd, stack = env
    ring = kvd.Ring(1, 1 << 30)
    a = np.zeros(4096, dtype=np.uint8)
    dev = torch.device("cuda:0")
    ok = torch.empty(4096, dtype=torch.uint8, device=dev)
    with pytest.raises(kvd.KvdError) as e:
        ring.stage(0, kvd.STAGE_ACQUIRE, a.ctypes.data, a.ctypes.data, 1088, 2, 1, 2, ok.data_ptr(), ok.data_ptr())
    assert e.value.code == kvd.KVD_EINVAL
    ring.close()


def test_cross_step_lookahead_is_bit_identical(env):
    """Prefetching the next step's first layers after the last layer of a step
    (their prefix is stable) changes nothing in the outputs."""
    torch, kvd, stack = env
    cfg = small_cfg()
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    ref, _ = run_arm(env, cfg, host, cfg.n_ctx, 0, 0, 3)
    for depth in (1, 3):
        st = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, depth, 1 << 30, new_rows=stack.token_rows(cfg),
                         cross_step=True)
        outs = []
        for t in range(3):
            st.token(t)
            with torch.cuda.stream(st.stream):
                outs.append([o.clone() for o in st.out])
        s = st.ring.stats()
        st.close()
        # steps after the first start from the deliveries issued at the end of the previous step
        assert s["n_acquire_primed"] == 0 and s["n_acquire_pipelined"] == 3 * cfg.n_layers
        assert s["n_prefetch"] == 3 * cfg.n_layers + depth   # the last step's look-ahead is never consumed
        for t in range(3):
            for l in range(cfg.n_layers):
                assert torch.equal(outs[t][l], ref[t][l]), (depth, t, l)
    host.free()
