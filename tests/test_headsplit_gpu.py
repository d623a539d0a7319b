"""GPU tests of the per-head residency split: KV heads [0, hr) device-resident,
the rest staged through the ring; each layer's output (two calls over
disjoint head ranges) against the oracle on the whole rows, and the
pipelined arm bit-identical to the ordered arm."""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _checker(oracle, errs, layers):
    def check(st, kv):
        g = np.random.default_rng([st.cfg.seed, 7777])
        qs = [g.standard_normal((1, st.cfg.n_head_q, st.cfg.head_dim)).astype(np.float32) for _ in range(kv.n_layers)]
        for l in layers:
            k, v = kv.full_rows(l)
            ref = oracle.attend(qs[l], [[(k, v, 0)]], st.cfg.n_head_kv, st.cfg.head_dim, threads=8)
            errs.append((l, float(np.abs(st.out[l].cpu().numpy() - ref).max())))
    return check


@pytest.mark.parametrize("hr", [0, 3, 5, 8])
def test_head_split_matches_oracle_and_ordered(oracle, hr):
    import torch
    from decode_attention_offloaded_amd import headsplit, kvd
    cfg = inputs.Config(94, "headsplit_test", 5, 1, 3000, 40, 8, 128)
    errs = []
    res = headsplit.run_headsplit(torch, kvd, inputs, cfg, hr, n_layers=cfg.n_layers, depths=(0, 1, 2),
                                  budget_bytes=1 << 30, tokens=2, warmup=1, gemv=False,
                                  check=_checker(oracle, errs, (0, cfg.n_layers - 1)), log=lambda *a: None)
    assert res["bit_identical"]
    assert len(errs) == 2
    for l, e in errs:
        assert e <= TOL, (hr, l, e)
    if hr < 8:
        for d in ("1", "2"):
            a = res["arms"][d]
            assert a["n_acquire_ordered"] == 0 and a["n_acquire_pipelined"] == 3 * cfg.n_layers, a
            assert a["ring_engaged_bytes"] == (int(d) + 2) * 2 * 3000 * (8 - hr) * 136
    else:
        assert res["staged_bytes_per_token"] == 0
