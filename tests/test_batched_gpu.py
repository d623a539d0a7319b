"""GPU tests of the batched mixed-residency stack: 16 sequences of lognormal
lengths, full-attention even layers and sliding-window odd layers, the older
half of every sequence staged from pinned host memory through the ring and
the newer half on the device, the two segments merged by the combine.
Checks: every layer's output against the oracle, and the pipelined arm
bit-identical to the ordered arm."""
import os

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    from decode_attention_offloaded_amd import batched, kvd
    return torch, kvd, batched


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _check_all_layers(oracle, errs):
    def check(st, lay, kv):
        for l in range(lay.n_layers):
            segs = kv.oracle_segments(l)
            ref = oracle.attend(st.q[l].cpu().numpy(), segs, st.cfg.n_head_kv, st.cfg.head_dim,
                                window=lay.window[l], q_pos=lay.q_pos, threads=_threads())
            got = st.out[l].cpu().numpy().astype(np.float64)
            errs.append((l, float(np.abs(got - ref.astype(np.float32)).max())))
    return check


def _run(env, oracle, lengths, n_layers, window):
    torch, kvd, batched = env
    cfg = inputs.config(4)
    errs = []
    res = batched.run_batched(torch, kvd, inputs, cfg, lengths=lengths, n_layers=n_layers, depths=(0, 1),
                              budget_bytes=1 << 30, tokens=1, warmup=1, gemm=False, window=window,
                              check=_check_all_layers(oracle, errs), log=lambda *a: None)
    return res, errs


def test_batched_small_matches_oracle_and_ordered(env, oracle):
    cfg = inputs.config(4)
    _, _, batched = env
    lengths = batched.cfg4_lengths(cfg, median=512, lo=64, hi=4096)
    res, errs = _run(env, oracle, lengths, 6, 512)
    assert res["bit_identical"]
    a1 = res["arms"]["1"]
    assert a1["declined"] == 0 and a1["n_acquire_ordered"] == 0 and a1["n_acquire_pipelined"] > 0, a1
    assert res["arms"]["0"]["n_acquire_ordered"] > 0
    assert len(errs) == 6
    for l, e in errs:
        assert e <= TOL, (l, e)


def test_batched_full_lengths_two_layers(env, oracle):
    """The batched workload's own lengths (lognormal around 4096, clipped to
    [1024, 32768]) and 4096-row window, on one full and one window layer."""
    cfg = inputs.config(4)
    _, _, batched = env
    lengths = batched.cfg4_lengths(cfg)
    res, errs = _run(env, oracle, lengths, 2, 4096)
    assert res["bit_identical"]
    assert len(errs) == 2
    for l, e in errs:
        assert e <= TOL, (l, e)


def test_window_layer_with_nothing_staged(env, oracle):
    """Every sequence at least twice the window: the odd layer stages no host
    row at all (no ACQUIRE), its host segments are empty, and the output
    still matches the oracle."""
    _, _, batched = env
    res, errs = _run(env, oracle, [300, 257, 1000, 512], 2, 128)
    assert res["arms"]["1"]["n_acquire_pipelined"] + res["arms"]["1"]["n_acquire_primed"] >= 1
    assert res["bit_identical"]
    for l, e in errs:
        assert e <= TOL, (l, e)
