"""GPU parity of the asymmetric cache: q8_0 K with q4_0 V (18-byte blocks),
against the fp64 oracle's q4_0 path (max abs error <= 1e-3), through the C
ABI; and through the staging ring (V rows staged at their own size), with the
pipelined path bit-identical to the ordered path."""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _cache(seed, n, hkv, d, vpad=0):
    rng = np.random.default_rng(seed)
    k = inputs.random_kv_rows(rng, n, hkv, d)
    v = inputs.random_kv_rows_q4_0(rng, n, hkv, d)
    if vpad:
        v = np.concatenate([v, rng.integers(0, 256, (n, vpad), dtype=np.uint8)], axis=1)
    return rng, k, v


def _gpu(q, segs, hkv, window=0, q_pos=None, split_rows=0):
    import torch
    from decode_attention_offloaded_amd import kvd
    qd = to_dev(q)
    out = torch.full_like(qd, float("nan"))
    dsegs = [[(to_dev(k), to_dev(v), p0) for (k, v, p0) in seq] for seq in segs]
    kvd.attend_decode(qd, out, dsegs, hkv, window=window, q_pos=q_pos, split_rows=split_rows,
                      v_type=kvd.TYPE_Q4_0)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,hq,hkv", [(128, 40, 8), (64, 8, 2), (128, 8, 8), (64, 16, 2), (128, 24, 4)])
@pytest.mark.parametrize("n", [1, 63, 65, 777, 4096])
def test_q4_v_matches_oracle(oracle, d, hq, hkv, n):
    rng, k, v = _cache(d * 100 + n + hq, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    got = _gpu(q, [[(k, v, 0)]], hkv)
    ref = oracle.attend(q, [[(k, v, 0)]], hkv, d, v_type=oracle.V_Q4_0, threads=8)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= TOL


@pytest.mark.parametrize("g_size", [5, 8])
def test_q4_v_long_context_every_head(oracle, g_size):
    """131072 rows x 8 KV heads with q4_0 V (one 12-wave workgroup per CU):
    the whole output against the oracle."""
    n, hkv, d = 131072, 8, 128
    hq = hkv * g_size
    rng, k, v = _cache(515 + g_size, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    got = _gpu(q, [[(k, v, 0)]], hkv)
    assert np.isfinite(got).all()
    ref = oracle.attend(q, [[(k, v, 0)]], hkv, d, v_type=oracle.V_Q4_0, threads=8)
    assert np.abs(got - ref).max() <= TOL


def test_q4_v_one_row_is_exact(oracle):
    rng, k, v = _cache(5, 1, 8, 128)
    q = inputs.random_q(rng, 1, 40, 128)
    got = _gpu(q, [[(k, v, 0)]], 8)
    vals = oracle.dequant_q4_0(v[0]).reshape(8, 128)
    for h in range(40):
        assert np.array_equal(got[0, h], vals[h // 5].astype(np.float32)), h


def test_q4_v_batch_two_segments_windows_and_padding(oracle):
    rng = np.random.default_rng(77)
    segs, lens = [], [300, 1000, 2500, 64]
    for i, n in enumerate(lens):
        _, k, v = _cache(100 + i, n, 8, 128, vpad=8 * (i % 2))
        h = n // 2
        segs.append([(k[:h], v[:h], 0), (k[h:], v[h:], h)])
    q = inputs.random_q(rng, len(lens), 40, 128)
    for window in (0, 700):
        got = _gpu(q, segs, 8, window=window)
        ref = oracle.attend(q, segs, 8, 128, window=window, v_type=oracle.V_Q4_0, threads=8)
        assert np.abs(got - ref).max() <= TOL, window


@pytest.mark.parametrize("split_rows", [64, 192, 1024, 8192])
def test_q4_v_split_sweep(oracle, split_rows):
    rng, k, v = _cache(9, 5000, 8, 128)
    q = inputs.random_q(rng, 1, 40, 128)
    got = _gpu(q, [[(k, v, 0)]], 8, split_rows=split_rows)
    ref = oracle.attend(q, [[(k, v, 0)]], 8, 128, v_type=oracle.V_Q4_0, threads=8)
    assert np.abs(got - ref).max() <= TOL


def test_q4_v_through_the_ring_bit_identical(oracle):
    import torch
    from decode_attention_offloaded_amd import kvd, stack
    cfg = inputs.Config(93, "q4v_ring_test", 8, 1, 3000, 40, 8, 128)
    vrb = inputs.row_bytes_q4_0(8, 128)
    host = stack.HostKV(cfg.n_layers, cfg.n_ctx, cfg.row_bytes, vrb, kvd.TYPE_Q4_0)
    host.fill(inputs, cfg, cfg.n_ctx)
    outs, stats = {}, {}
    for depth in (0, 1, 2):
        st = stack.Stack(torch, kvd, cfg, host, cfg.n_ctx, depth, 1 << 30,
                         new_rows=stack.token_rows(cfg, v_type=kvd.TYPE_Q4_0))
        for t in range(2):
            st.token(t)
        outs[depth] = [o.clone() for o in st.out]
        stats[depth] = st.ring.stats()
        st.close()
    for depth in (1, 2):
        assert stats[depth]["n_acquire_ordered"] == 0, stats[depth]
        assert stats[depth]["ring_bytes"] == (depth + 2) * cfg.n_ctx * (cfg.row_bytes + vrb)
        for a, b in zip(outs[0], outs[depth]):
            assert torch.equal(a, b)
    assert stats[1]["bytes_early"] == 2 * cfg.n_layers * (cfg.n_ctx - 1) * (cfg.row_bytes + vrb)
    g = np.random.default_rng([cfg.seed, 7777])
    qs = [g.standard_normal((1, 40, 128)).astype(np.float32) for _ in range(cfg.n_layers)]
    for l in (0, cfg.n_layers - 1):
        ref = oracle.attend(qs[l], [[(host.k_rows(l).copy(), host.v_rows(l).copy(), 0)]], 8, 128,
                            v_type=oracle.V_Q4_0, threads=8)
        assert np.abs(outs[0][l].cpu().numpy() - ref).max() <= TOL
    host.free()
