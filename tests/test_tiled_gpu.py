"""GPU tests of tile-streamed attention: per-tile partial results merged by
kvd_attend_merge must equal attention over the whole row set (oracle within
1e-3; the direct call within float rounding), and a tile-streamed stack must
give bit-identical outputs ordered and pipelined, including at a budget where
a whole-layer ring declines."""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from tests.helpers import make_cache

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    from decode_attention_offloaded_amd import kvd, stack, tiled
    return torch, kvd, stack, tiled


def _tiles_attend(torch, kvd, q, k, v, bounds, n_head_kv, window=0):
    """Per-tile partial calls over [bounds[i], bounds[i+1]) then one merge."""
    n_seq, hq, d = q.shape
    pf = kvd.partial_floats(n_seq, hq, d)
    qd = torch.from_numpy(q).cuda()
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    parts = torch.full(((len(bounds) - 1) * pf,), float("nan"), dtype=torch.float32, device="cuda")
    qpos = [k.shape[0] - 1] * n_seq
    for i in range(len(bounds) - 1):
        r0, r1 = bounds[i], bounds[i + 1]
        seg = (kd[r0:r1], vd[r0:r1], r0)
        kvd.attend_decode_partial(qd, parts[i * pf:(i + 1) * pf], [[seg]] * n_seq, n_head_kv, window=window,
                                  q_pos=qpos)
    out = torch.full_like(qd, float("nan"))
    kvd.attend_merge(parts, len(bounds) - 1, out)
    direct = torch.full_like(qd, float("nan"))
    kvd.attend_decode(qd, direct, [[(kd, vd, 0)]] * n_seq, n_head_kv, window=window, q_pos=qpos)
    torch.cuda.synchronize()
    return out.cpu().numpy(), direct.cpu().numpy()


@pytest.mark.parametrize("d,hq,hkv", [(128, 40, 8), (64, 8, 2), (128, 16, 16)])
@pytest.mark.parametrize("bounds", [[0, 5000], [0, 1000, 1063, 3000, 5000], [0, 1, 64, 4999, 5000]])
def test_partials_merge_to_the_whole(env, oracle, d, hq, hkv, bounds):
    torch, kvd, _, _ = env
    _, k, v = make_cache(11 + len(bounds), 5000, hkv, d)
    q = inputs.random_q(np.random.default_rng(3), 2, hq, d)
    got, direct = _tiles_attend(torch, kvd, q, k, v, bounds, hkv)
    ref = oracle.attend(q, [[(k, v, 0)]] * 2, hkv, d, threads=8)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= TOL
    assert np.abs(got - direct).max() <= 2e-5


def test_partials_with_a_window(env, oracle):
    torch, kvd, _, _ = env
    _, k, v = make_cache(5, 3000, 8, 128)
    q = inputs.random_q(np.random.default_rng(4), 1, 40, 128)
    # window 1500: rows [1500, 3000) visible; every tile keeps a visible row
    got, direct = _tiles_attend(torch, kvd, q, k, v, [0, 1600, 2000, 3000], 8, window=1500)
    ref = oracle.attend(q, [[(k, v, 0)]], 8, 128, window=1500, threads=8)
    assert np.abs(got - ref).max() <= TOL
    assert np.abs(got - direct).max() <= 2e-5
    # a tile with no visible row is an error, reported before anything runs
    with pytest.raises(kvd.KvdError):
        _tiles_attend(torch, kvd, q, k, v, [0, 1000, 3000], 8, window=1500)


def _small_cfg():
    return inputs.Config(91, "tiled_test", 6, 1, 3000, 40, 8, 128)


def _oracle_check(oracle, cfg, host, outs, n_rows):
    g = np.random.default_rng([cfg.seed, 7777])
    qs = [g.standard_normal((1, cfg.n_head_q, cfg.head_dim)).astype(np.float32) for _ in range(host.n_layers)]
    for l in (0, host.n_layers - 1):
        k = host.k_rows(l)[:n_rows].copy()
        v = host.v_rows(l)[:n_rows].copy()
        ref = oracle.attend(qs[l], [[(k, v, 0)]], cfg.n_head_kv, cfg.head_dim, threads=8)
        assert np.abs(outs[l].cpu().numpy() - ref).max() <= TOL, l


def test_tiled_stack_bit_identical_and_oracle(env, oracle):
    torch, kvd, stack, tiled = env
    cfg = _small_cfg()
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    res = tiled.run_tiled(torch, kvd, inputs, cfg, n_layers=cfg.n_layers, depths=(0, 1, 2), budget_bytes=1 << 30,
                          tile_rows=640, tokens=2, warmup=1, gemv=False, host=host, log=lambda *a: None)
    assert res["tiles_per_layer"] == 5 and res["bit_identical"]
    for d in ("1", "2"):
        a = res["arms"][d]
        assert a["declined"] == 0 and a["n_acquire_ordered"] == 0 and a["n_acquire_pipelined"] > 0, a
    assert res["arms"]["0"]["n_acquire_ordered"] == 3 * cfg.n_layers * 5
    _oracle_check(oracle, cfg, host, res["outs"], cfg.n_ctx)
    host.free()


def test_tiles_engage_where_a_whole_layer_ring_declines(env, oracle):
    torch, kvd, stack, tiled = env
    cfg = _small_cfg()
    budget = 8 << 20   # a whole 3000-row layer needs 3 x 2 x 3000 x 1088 = 19.6 MB at depth 1
    rc, rows = kvd.tile_rows(1, budget, cfg.row_bytes)
    assert rc == kvd.KVD_OK and rows == 1280
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes)
    host.fill(inputs, cfg, cfg.n_ctx)
    whole = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, 1, budget)
    whole.token(0)
    s = whole.ring.stats()
    whole.close()
    assert s["declined"] == 1 and s["n_acquire_ordered"] == cfg.n_layers
    res = tiled.run_tiled(torch, kvd, inputs, cfg, n_layers=cfg.n_layers, depths=(0, 1), budget_bytes=budget,
                          tokens=1, warmup=1, gemv=False, host=host, log=lambda *a: None)
    assert res["tile_rows"] == 1280 and res["tiles_per_layer"] == 3 and res["bit_identical"]
    a = res["arms"]["1"]
    assert a["declined"] == 0 and a["n_acquire_pipelined"] == 2 * 3 * cfg.n_layers
    assert a["ring_engaged_bytes"] <= budget
    _oracle_check(oracle, cfg, host, res["outs"], cfg.n_ctx)
    host.free()
