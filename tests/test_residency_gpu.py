"""GPU test of partial device residency: a resident prefix of layers plus the
rest staged (ring or ordered) gives outputs bit-identical to staging every
layer, and the resident layers are never staged."""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

pytestmark = pytest.mark.gpu


def test_resident_prefix_is_bit_identical_to_staging(oracle):
    import torch
    from decode_attention_offloaded_amd import kvd, stack
    cfg = inputs.Config(92, "residency_test", 12, 1, 3000, 40, 8, 128)
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    arms = [("ring", 1, 1 << 30, 0), ("ring+3", 1, 1 << 30, 3), ("ordered+5", 0, 0, 5), ("resident", 0, 0, 12)]
    res = stack.run_residency(torch, kvd, inputs, cfg, arms, n_layers=cfg.n_layers, tokens=2, warmup=1,
                              host=host, log=lambda *a: None)
    assert res["bit_identical"]
    a = res["arms"]
    assert a["ring"]["n_acquire_pipelined"] == 3 * 12 and a["ring"]["n_acquire_ordered"] == 0
    assert a["ring+3"]["n_acquire_pipelined"] == 3 * 9 and a["ring+3"]["n_acquire_ordered"] == 0
    assert a["ordered+5"]["n_acquire_ordered"] == 3 * 7 and a["ordered+5"]["n_acquire_pipelined"] == 0
    assert a["resident"]["n_acquire_ordered"] == 0 and a["resident"]["n_acquire_pipelined"] == 0
    # and one resident and one staged layer against the oracle (last token's rows)
    st = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, 0, 0, resident=3)
    st.token(99)
    for l in (1, 7):
        k = host.k_rows(l)[:cfg.n_ctx].copy()
        v = host.v_rows(l)[:cfg.n_ctx].copy()
        ref = oracle.attend(st.q[l].cpu().numpy(), [[(k, v, 0)]], cfg.n_head_kv, cfg.head_dim, threads=8)
        assert np.abs(st.out[l].cpu().numpy() - ref).max() <= 1e-3, l
    st.close()
    host.free()
