"""Full-size host-resident stacks in the launch configurations the benchmark
times, every output of the checked layers against the oracle:
- 16384 rows through a depth-1 ring of 128 MiB (whole layers);
- 131072 rows at 128 MiB, where a whole-layer ring declines and the layer
  is streamed in tiles through the ring;
- 131072 rows through a depth-1 ring of 1 GiB (whole layers).
Ordered and pipelined arms must agree bit for bit."""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from tests.helpers import head_slice

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _qs(cfg, n_layers):
    g = np.random.default_rng([cfg.seed, 7777])
    return [g.standard_normal((1, cfg.n_head_q, cfg.head_dim)).astype(np.float32) for _ in range(n_layers)]


def _check_layer(oracle, cfg, host, l, q, out, heads=None):
    n = host.cap_rows
    k, v = host.k_rows(l)[:n], host.v_rows(l)[:n]
    G = cfg.n_head_q // cfg.n_head_kv
    got = out.cpu().numpy()
    if heads is None:
        ref = oracle.attend(q, [[(k.copy(), v.copy(), 0)]], cfg.n_head_kv, cfg.head_dim, threads=16)
        assert np.abs(got - ref).max() <= TOL
        return
    for g in heads:
        ks, vs = head_slice(k, g, cfg.n_head_kv, cfg.head_dim), head_slice(v, g, cfg.n_head_kv, cfg.head_dim)
        ref = oracle.attend(q[:, g * G:(g + 1) * G], [[(ks, vs, 0)]], 1, cfg.head_dim, threads=16)
        assert np.abs(got[:, g * G:(g + 1) * G] - ref).max() <= TOL, g


def test_16k_stack_128mib_ring(oracle):
    import torch
    from decode_attention_offloaded_amd import kvd, stack
    base = inputs.config(2)
    cfg = inputs.Config(2, base.name, 4, 1, base.n_ctx, base.n_head_q, base.n_head_kv, base.head_dim)
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    outs = {}
    for depth in (0, 1):
        st = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, depth, 128 << 20, new_rows=stack.token_rows(cfg))
        for t in range(2):
            st.token(t)
        s = st.ring.stats()
        outs[depth] = [o.clone() for o in st.out]
        st.close()
        if depth == 1:
            assert s["engaged"] == 1 and s["ring_bytes"] == 106_954_752 and s["n_acquire_ordered"] == 0
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    qs = _qs(cfg, cfg.n_layers)
    for l in (0, cfg.n_layers - 1):
        _check_layer(oracle, cfg, host, l, qs[l], outs[1][l])
    host.free()


def test_128k_tiled_at_128mib(oracle):
    import torch
    from decode_attention_offloaded_amd import kvd, stack, tiled
    base = inputs.config(3)
    cfg = inputs.Config(3, base.name, 2, 1, base.n_ctx, base.n_head_q, base.n_head_kv, base.head_dim)
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    res = tiled.run_tiled(torch, kvd, inputs, cfg, n_layers=cfg.n_layers, depths=(0, 1), budget_bytes=128 << 20,
                          tokens=1, warmup=1, gemv=False, host=host, log=lambda *a: None)
    assert res["tile_rows"] == 20544 and res["tiles_per_layer"] == 7 and res["bit_identical"]
    a = res["arms"]["1"]
    assert a["declined"] == 0 and a["n_acquire_ordered"] == 0 and a["ring_engaged_bytes"] == 134_111_232
    qs = _qs(cfg, cfg.n_layers)
    for l in range(cfg.n_layers):
        _check_layer(oracle, cfg, host, l, qs[l], res["outs"][l])
    host.free()


def test_128k_whole_layer_ring_at_1gib(oracle):
    import torch
    from decode_attention_offloaded_amd import kvd, stack
    base = inputs.config(3)
    cfg = inputs.Config(3, base.name, 2, 1, base.n_ctx, base.n_head_q, base.n_head_kv, base.head_dim)
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    outs = {}
    for depth, budget in ((0, 0), (1, 1 << 30), (2, 1 << 30)):
        st = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, depth, budget, new_rows=stack.token_rows(cfg))
        st.token(0)
        s = st.ring.stats()
        outs[depth] = [o.clone() for o in st.out]
        st.close()
        if depth == 1:
            assert s["engaged"] == 1 and s["ring_bytes"] == 855_638_016
        if depth == 2:
            assert s["declined"] == 1 and s["need_bytes"] == 1_140_850_688
    for d in (1, 2):
        for a, b in zip(outs[0], outs[d]):
            assert torch.equal(a, b)
    qs = _qs(cfg, cfg.n_layers)
    for l in range(cfg.n_layers):
        _check_layer(oracle, cfg, host, l, qs[l], outs[1][l])
    host.free()
