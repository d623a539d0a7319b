"""GPU parity: the HIP decode-attention kernel against the fp64 oracle.

Tolerance: max abs error <= 1e-3 against fp32(oracle) (the bar the build is
held to); observed errors are ~1e-6.  Exact cases (one visible row) must be
bit-exact.  All inputs are seeded and synthetic (decode_attention_offloaded_amd.inputs).
"""
import math

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from tests.helpers import gpu_attend, head_slice, make_cache, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-3


def check(out, ref, tol=TOL):
    assert np.all(np.isfinite(out)), "non-finite output"
    err = np.max(np.abs(out.astype(np.float64) - ref))
    assert err <= tol, "max abs error %.3g > %.3g" % (err, tol)
    return err


def test_config0_tiny(oracle):
    c = inputs.config(0)
    rng = c.layer_rng(0)
    k = inputs.random_kv_rows(rng, c.n_ctx, c.n_head_kv, c.head_dim)
    v = inputs.random_kv_rows(rng, c.n_ctx, c.n_head_kv, c.head_dim)
    q = inputs.random_q(rng, 1, c.n_head_q, c.head_dim)
    ref = oracle.attend(q, [[(k, v, 0)]], c.n_head_kv, c.head_dim)
    out = gpu_attend(q, [[(k, v, 0)]], c.n_head_kv)
    print("cfg0 err", check(out, ref))


def test_config1_full(oracle):
    c = inputs.config(1)
    rng = c.layer_rng(0)
    k = inputs.random_kv_rows(rng, c.n_ctx, c.n_head_kv, c.head_dim)
    v = inputs.random_kv_rows(rng, c.n_ctx, c.n_head_kv, c.head_dim)
    q = inputs.random_q(rng, 1, c.n_head_q, c.head_dim)
    ref = oracle.attend(q, [[(k, v, 0)]], c.n_head_kv, c.head_dim, threads=8)
    out = gpu_attend(q, [[(k, v, 0)]], c.n_head_kv)
    print("cfg1 err", check(out, ref))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (10, 2), (40, 8), (16, 2), (32, 32), (64, 16), (8, 1), (5, 1)])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 160, 200, 384, 777])
def test_shapes_and_ragged_tails(oracle, d, hq, hkv, n):
    rng, k, v = make_cache(1000 + n + d + hq, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    ref = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    out = gpu_attend(q, [[(k, v, 0)]], hkv)
    check(out, ref)


@pytest.mark.parametrize("d", [64, 128])
def test_single_row_is_bit_exact(oracle, d):
    """One visible row: weight e^0 / 1 = 1, so the output is d * code exactly."""
    hq, hkv = 8, 2
    rng, k, v = make_cache(7, 1, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    out = gpu_attend(q, [[(k, v, 0)]], hkv)
    vv = oracle.dequant_q8_0(v).reshape(1, hkv, d)[0].astype(np.float32)
    assert np.array_equal(out[0], vv[np.arange(hq) // (hq // hkv)])
    # also as the only visible row of a longer segment (window 1)
    rng, k, v = make_cache(8, 300, hkv, d)
    out = gpu_attend(q, [[(k, v, 0)]], hkv, window=1)
    vv = oracle.dequant_q8_0(v).reshape(300, hkv, d)[-1].astype(np.float32)
    assert np.array_equal(out[0], vv[np.arange(hq) // (hq // hkv)])


@pytest.mark.parametrize("split_rows", [64, 128, 256, 1024, 4096])
def test_split_sweep_config1(oracle, split_rows):
    c = inputs.config(1)
    rng = c.layer_rng(1)
    n = 3000  # ragged against every split size
    k = inputs.random_kv_rows(rng, n, c.n_head_kv, c.head_dim)
    v = inputs.random_kv_rows(rng, n, c.n_head_kv, c.head_dim)
    q = inputs.random_q(rng, 1, c.n_head_q, c.head_dim)
    ref = oracle.attend(q, [[(k, v, 0)]], c.n_head_kv, c.head_dim, threads=8)
    out = gpu_attend(q, [[(k, v, 0)]], c.n_head_kv, split_rows=split_rows)
    check(out, ref)
    one = gpu_attend(q, [[(k, v, 0)]], c.n_head_kv, split_rows=4096)
    assert np.max(np.abs(out - one)) < 1e-5


def test_row_stride_padding(oracle):
    hq, hkv, d, n = 40, 8, 128, 500
    rng, k, v = make_cache(9, n, hkv, d, pad=24)
    q = inputs.random_q(rng, 1, hq, d)
    ref = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    check(gpu_attend(q, [[(k, v, 0)]], hkv), ref)


def test_query_position_and_window(oracle):
    hq, hkv, d, n = 40, 8, 128, 1500
    rng, k, v = make_cache(10, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    for w, qp in [(0, 1000), (256, None), (256, 900), (1, 5), (5000, None)]:
        qpos = None if qp is None else [qp]
        ref = oracle.attend(q, [[(k, v, 40)]], hkv, d, window=w, q_pos=None if qp is None else [qp + 40])
        out = gpu_attend(q, [[(k, v, 40)]], hkv, window=w, q_pos=None if qp is None else [qp + 40])
        check(out, ref)


def test_batched_varlen_swa_two_segments(oracle):
    """A small version of the batched workload: lognormal lengths, the older
    half of every sequence in one segment and the newer half in another,
    full attention and a sliding window."""
    rng = np.random.default_rng(20264)
    hq, hkv, d = 40, 8, 128
    lens = inputs.lognormal_lengths(rng, 16, median=300, sigma=1.0, lo=60, hi=2400)
    q = inputs.random_q(rng, 16, hq, d)
    segs = []
    for i, n in enumerate(lens):
        k = inputs.random_kv_rows(rng, int(n), hkv, d)
        v = inputs.random_kv_rows(rng, int(n), hkv, d)
        h = int(n) // 2
        segs.append([(k[:h], v[:h], 0), (k[h:], v[h:], h)])
    for w in (0, 256):
        ref = oracle.attend(q, segs, hkv, d, window=w, threads=8)
        out = gpu_attend(q, segs, hkv, window=w)
        check(out, ref)


def test_one_workspace_for_calls_of_every_shape(oracle):
    """One workspace serves, in turn, a long single-sequence call, a
    16-sequence call in two segments, a call with other head counts and the
    first call again: whatever an earlier call left in it, each call's
    partials are its own."""
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(5150)
    ws = kvd.Workspace()
    calls = []
    k, v = inputs.random_kv_rows(rng, 9000, 8, 128), inputs.random_kv_rows(rng, 9000, 8, 128)
    calls.append((inputs.random_q(rng, 1, 40, 128), [[(k, v, 0)]], 8, 128))
    lens = inputs.lognormal_lengths(rng, 16, median=700, sigma=0.8, lo=200, hi=3000)
    segs = []
    for n in lens:
        kk, vv = inputs.random_kv_rows(rng, int(n), 8, 128), inputs.random_kv_rows(rng, int(n), 8, 128)
        h = int(n) // 2
        segs.append([(kk[:h], vv[:h], 0), (kk[h:], vv[h:], h)])
    calls.append((inputs.random_q(rng, 16, 40, 128), segs, 8, 128))
    k2, v2 = inputs.random_kv_rows(rng, 5000, 2, 64), inputs.random_kv_rows(rng, 5000, 2, 64)
    calls.append((inputs.random_q(rng, 1, 16, 64), [[(k2, v2, 0)]], 2, 64))
    calls.append(calls[0])
    import torch
    for q, sg, hkv, d in calls:
        ref = oracle.attend(q, sg, hkv, d, threads=8)
        qd = to_dev(q)
        out = torch.full_like(qd, float("nan"))
        kvd.attend_decode(qd, out, [[(to_dev(a), to_dev(b), p0) for (a, b, p0) in seq] for seq in sg], hkv,
                          workspace=ws)
        torch.cuda.synchronize()
        check(out.cpu().numpy(), ref)


def test_empty_first_segment_under_window(oracle):
    hq, hkv, d = 8, 2, 64
    rng, k, v = make_cache(11, 400, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    segs = [[(k[:200], v[:200], 0), (k[200:], v[200:], 200)]]
    ref = oracle.attend(q, segs, hkv, d, window=100)
    check(gpu_attend(q, segs, hkv, window=100), ref)


def test_deterministic_and_pointer_independent():
    import torch
    hq, hkv, d, n = 40, 8, 128, 5000
    rng, k, v = make_cache(12, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    a = gpu_attend(q, [[(k, v, 0)]], hkv)
    b = gpu_attend(q, [[(k.copy(), v.copy(), 0)]], hkv)
    c = gpu_attend(q, [[(k, v, 0)]], hkv)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_sequence_order_does_not_change_any_output(oracle):
    """A launch fills its slots longest sequence first and each slot carries
    its sequence's query/output index: the same 16 sequences (two segments
    each, lengths 300 ... 9000 rows) given in reverse order give every
    sequence's output bit for bit, and the output matches the oracle."""
    hq, hkv, d = 40, 8, 128
    rng = np.random.default_rng(1616)
    lens = [300, 9000, 1200, 4100, 700, 6400, 2500, 8000, 1024, 3333, 5000, 450, 7777, 2048, 6100, 999]
    segs = []
    for n in lens:
        k = inputs.random_kv_rows(rng, n, hkv, d)
        v = inputs.random_kv_rows(rng, n, hkv, d)
        h = n // 2
        segs.append([(k[:h], v[:h], 0), (k[h:], v[h:], h)])
    q = inputs.random_q(rng, len(lens), hq, d)
    fwd = gpu_attend(q, segs, hkv)
    rev = gpu_attend(q[::-1].copy(), segs[::-1], hkv)
    assert np.array_equal(fwd, rev[::-1])
    ref = oracle.attend(q, segs, hkv, d, threads=8)
    check(fwd, ref)


def test_long_context_every_head(oracle):
    """131072 rows x 40/8 heads (the long-context layer, one 12-wave
    workgroup per CU, 32 splits per KV head): the whole output against the
    oracle (about a second of fp64 on 8 threads)."""
    c = inputs.config(3)
    rng = c.layer_rng(0)
    n = c.n_ctx
    k = inputs.random_kv_rows(rng, n, c.n_head_kv, c.head_dim)
    v = inputs.random_kv_rows(rng, n, c.n_head_kv, c.head_dim)
    q = inputs.random_q(rng, 1, c.n_head_q, c.head_dim)
    out = gpu_attend(q, [[(k, v, 0)]], c.n_head_kv)
    ref = oracle.attend(q, [[(k, v, 0)]], c.n_head_kv, c.head_dim, threads=8)
    check(out, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g_size", [1, 2, 4, 8])
def test_long_range_every_group_size(oracle, d, g_size):
    """One range of 65600 rows x 8 KV heads (ragged last sub-tile), three
    ways: as planned (one 12-wave workgroup per CU), in 2112-row splits (32
    per KV head) and in two segments.  Sampled KV heads of each against the
    oracle, for group sizes 1 (15 padding columns in every MFMA) up to 8."""
    n, hkv = 65600, 8
    hq = hkv * g_size
    rng, k, v = make_cache(7000 + d + g_size, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    one = gpu_attend(q, [[(k, v, 0)]], hkv)
    wide = gpu_attend(q, [[(k, v, 0)]], hkv, split_rows=2112)
    h = n // 3
    two = gpu_attend(q, [[(k[:h], v[:h], 0), (k[h:], v[h:], h)]], hkv)
    for g in (1, hkv - 2):
        ks, vs = head_slice(k, g, hkv, d), head_slice(v, g, hkv, d)
        ref = oracle.attend(q[:, g * g_size:(g + 1) * g_size], [[(ks, vs, 0)]], 1, d, threads=8)
        for out in (one, wide, two):
            check(out[:, g * g_size:(g + 1) * g_size], ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("v_type", [0, 1])
def test_eight_wave_workgroups(oracle, d, v_type):
    """20001 rows x 8 KV heads: enough work per CU for 8-wave workgroups (one
    per CU), q8_0 and q4_0 V, as planned, in 640-row splits and in two
    segments; sampled KV heads against the oracle."""
    from decode_attention_offloaded_amd import kvd
    n, hkv, g_size = 20001, 8, 5
    hq = hkv * g_size
    rng = np.random.default_rng(8100 + d + v_type)
    k = inputs.random_kv_rows(rng, n, hkv, d)
    v = inputs.random_kv_rows_q4_0(rng, n, hkv, d) if v_type else inputs.random_kv_rows(rng, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    import torch
    qd = to_dev(q)
    h = n // 3
    outs = []
    for segs, sr in (([(k, v, 0)], 0), ([(k, v, 0)], 640), ([(k[:h], v[:h], 0), (k[h:], v[h:], h)], 0)):
        out = torch.full_like(qd, float("nan"))
        kvd.attend_decode(qd, out, [[(to_dev(a), to_dev(b), p0) for (a, b, p0) in segs]], hkv, split_rows=sr,
                          v_type=v_type)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    kcb, vcb = d // 32 * 34, d // 32 * (18 if v_type else 34)
    for g in (0, 6):
        ks = np.ascontiguousarray(k[:, g * kcb:(g + 1) * kcb])
        vs = np.ascontiguousarray(v[:, g * vcb:(g + 1) * vcb])
        ref = oracle.attend(q[:, g * g_size:(g + 1) * g_size], [[(ks, vs, 0)]], 1, d, threads=8,
                            v_type=oracle.V_Q4_0 if v_type else oracle.V_Q8_0)
        for out in outs:
            check(out[:, g * g_size:(g + 1) * g_size], ref)


@pytest.mark.parametrize("n,v_type", [(4096, 0), (300, 0), (200000 // 64 * 64, 0), (4096, 1)])
def test_graph_replays_match_eager(n, v_type):
    """Decode attention captured in a HIP graph (decode and combine launches,
    no memset nodes) and replayed several times, with eager work and
    synchronisations in between: every replay equals the eager call bit for
    bit, and the partial/merge pair captures the same way."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(n + v_type)
    k = inputs.random_kv_rows(rng, n, 8, 128)
    v = inputs.random_kv_rows_q4_0(rng, n, 8, 128) if v_type else inputs.random_kv_rows(rng, n, 8, 128)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    q = torch.from_numpy(inputs.random_q(rng, 1, 40, 128)).cuda()
    ws = kvd.Workspace()
    s = torch.cuda.Stream()
    eager = torch.empty_like(q)
    with torch.cuda.stream(s):
        kvd.attend_decode(q, eager, [[(kd, vd, 0)]], 8, workspace=ws, stream=s, v_type=v_type)
    torch.cuda.synchronize()
    out = torch.full_like(q, float("nan"))
    pf = kvd.partial_floats(1, 40, 128)
    parts = torch.empty(2 * pf, dtype=torch.float32, device="cuda")
    merged = torch.full_like(q, float("nan"))
    h = n // 2
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kvd.attend_decode(q, out, [[(kd, vd, 0)]], 8, workspace=ws, stream=s, v_type=v_type)
        kvd.attend_decode_partial(q, parts[:pf], [[(kd[:h], vd[:h], 0)]], 8, q_pos=[n - 1], workspace=ws,
                                  stream=s, v_type=v_type)
        kvd.attend_decode_partial(q, parts[pf:], [[(kd[h:], vd[h:], h)]], 8, q_pos=[n - 1], workspace=ws,
                                  stream=s, v_type=v_type)
        kvd.attend_merge(parts, 2, merged, stream=s)
    first_merged = None
    for rep in range(4):
        out.fill_(float("nan"))
        merged.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        if first_merged is None:
            first_merged = merged.clone()
            assert (first_merged - eager).abs().max().item() <= 2e-5
        assert torch.equal(merged, first_merged), rep
        # eager work between replays
        tmp = torch.empty_like(q)
        kvd.attend_decode(q, tmp, [[(kd, vd, 0)]], 8, v_type=v_type)
        torch.cuda.synchronize()


def test_workspace_grows_eagerly_and_under_capture():
    """A workspace sized by a short call grows for larger ones: between eager
    calls (after a device wait: 1024 rows, then 8192, in 64-row splits) and
    during graph capture (keeping the old buffer: 8192 rows with 64 query
    heads, more partials per split).  Outputs equal those of calls with a fresh
    workspace of their own, and the captured call replays to the same bytes."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(4321)

    def cache(n, hq):
        kd = torch.from_numpy(inputs.random_kv_rows(rng, n, 8, 128)).cuda()
        vd = torch.from_numpy(inputs.random_kv_rows(rng, n, 8, 128)).cuda()
        return torch.from_numpy(inputs.random_q(rng, 1, hq, 128)).cuda(), [[(kd, vd, 0)]]

    calls = [cache(1024, 40), cache(8192, 40), cache(8192, 64)]
    refs = []
    for q, segs in calls:
        r = torch.empty_like(q)
        kvd.attend_decode(q, r, segs, 8, workspace=kvd.Workspace(), split_rows=64)
        refs.append(r)
    torch.cuda.synchronize()
    ws = kvd.Workspace()
    s = torch.cuda.Stream()
    sizes = []
    with torch.cuda.stream(s):
        for (q, segs), ref in zip(calls[:2], refs[:2]):   # grows between eager calls
            out = torch.empty_like(q)
            kvd.attend_decode(q, out, segs, 8, workspace=ws, stream=s, split_rows=64)
            s.synchronize()
            assert torch.equal(out, ref)
            sizes.append(ws._buf[torch.cuda.current_device()].numel())
    q, segs = calls[2]
    out = torch.full_like(q, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):                     # grows during capture
        kvd.attend_decode(q, out, segs, 8, workspace=ws, stream=s, split_rows=64)
    sizes.append(ws._buf[torch.cuda.current_device()].numel())
    assert sizes[0] < sizes[1] < sizes[2], sizes
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[2]), rep


def test_captured_workspace_survives_eager_growth():
    """A graph captured with a workspace keeps writing its split partials into
    that buffer on every replay.  Growing the workspace afterwards (an eager
    call needing more) must not hand that buffer back to the allocator: a
    tensor allocated next must not share it, and replays must still equal the
    eager result."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(777)

    def cache(n):
        kd = torch.from_numpy(inputs.random_kv_rows(rng, n, 8, 128)).cuda()
        vd = torch.from_numpy(inputs.random_kv_rows(rng, n, 8, 128)).cuda()
        return torch.from_numpy(inputs.random_q(rng, 1, 40, 128)).cuda(), [[(kd, vd, 0)]]

    small, big = cache(2048), cache(8192)   # in 64-row splits: 32 and 128 per KV head
    ref = torch.empty_like(small[0])
    kvd.attend_decode(small[0], ref, small[1], 8, workspace=kvd.Workspace(), split_rows=64)
    torch.cuda.synchronize()
    ws = kvd.Workspace()
    s = torch.cuda.Stream()
    out = torch.full_like(small[0], float("nan"))
    with torch.cuda.stream(s):
        kvd.attend_decode(small[0], out, small[1], 8, workspace=ws, stream=s, split_rows=64)   # sizes the workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kvd.attend_decode(small[0], out, small[1], 8, workspace=ws, stream=s, split_rows=64)
    captured = ws._buf[torch.cuda.current_device()]
    cap_ptr, cap_len = captured.data_ptr(), captured.numel()
    del captured
    big_out = torch.empty_like(big[0])
    kvd.attend_decode(big[0], big_out, big[1], 8, workspace=ws, split_rows=64)            # grows the workspace eagerly
    torch.cuda.synchronize()
    assert ws._buf[torch.cuda.current_device()].data_ptr() != cap_ptr
    fillers = [torch.full((cap_len // 4,), 7.0, dtype=torch.float32, device="cuda") for _ in range(4)]
    for f in fillers:
        lo, hi = f.data_ptr(), f.data_ptr() + f.numel() * 4
        assert hi <= cap_ptr or lo >= cap_ptr + cap_len, "a new tensor reuses the captured workspace"
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        for f in fillers:
            assert bool((f == 7.0).all()), rep


@pytest.mark.parametrize("v_type", [0, 1])
def test_more_sequences_than_one_launch(oracle, v_type):
    """37 sequences: the call is split into launches of 16 sequences; outputs,
    split partials and the partial-result layout must all line up across
    launches (also through kvd_attend_decode_partial + kvd_attend_merge)."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(37 + v_type)
    lens = rng.integers(1, 900, size=37)
    lens[5] = 3000   # one long sequence: several splits in the middle launch
    vgen = inputs.random_kv_rows_q4_0 if v_type else inputs.random_kv_rows
    segs_np = []
    for n in lens:
        segs_np.append([(inputs.random_kv_rows(rng, int(n), 2, 64), vgen(rng, int(n), 2, 64), 0)])
    q = inputs.random_q(rng, 37, 8, 64)
    qd = torch.from_numpy(q).cuda()
    dsegs = [[(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), p0) for (k, v, p0) in s] for s in segs_np]
    out = torch.full_like(qd, float("nan"))
    kvd.attend_decode(qd, out, dsegs, 2, v_type=v_type)
    pf = kvd.partial_floats(37, 8, 64)
    parts = torch.empty(2 * pf + 4, dtype=torch.float32, device="cuda")
    # two "tiles": the first half of every sequence's rows, then the rest
    first = [[(k[:max(1, k.shape[0] // 2)], v[:max(1, k.shape[0] // 2)], 0)] for ((k, v, _),) in dsegs]
    rest = [[(k[max(1, k.shape[0] // 2):], v[max(1, k.shape[0] // 2):], max(1, k.shape[0] // 2))]
            for ((k, v, _),) in dsegs]
    qpos = [int(n) - 1 for n in lens]
    one_row = [i for i, n in enumerate(lens) if n == 1]
    merged = torch.full_like(qd, float("nan"))
    if not one_row:
        kvd.attend_decode_partial(qd, parts[:pf], first, 2, q_pos=qpos, v_type=v_type)
        kvd.attend_decode_partial(qd, parts[pf:2 * pf], rest, 2, q_pos=qpos, v_type=v_type)
        kvd.attend_merge(parts[:2 * pf], 2, merged)
    torch.cuda.synchronize()
    ref = oracle.attend(q, segs_np, 2, 64, threads=8, v_type=oracle.V_Q4_0 if v_type else oracle.V_Q8_0)
    got = out.cpu().numpy()
    assert np.abs(got - ref).max() <= 1e-3
    if not one_row:
        assert np.abs(merged.cpu().numpy() - ref).max() <= 1e-3


def _plan_of(q, segs_np, n_head_kv):
    """(split rows, waves, total splits) that a call with these shapes gets."""
    import torch
    from decode_attention_offloaded_amd import kvd
    qd = to_dev(q)
    segs = [[(to_dev(k[:1]), to_dev(v[:1]), p0) for (k, v, p0) in seq] for seq in segs_np]
    a, keep = kvd.make_args(qd, torch.empty_like(qd), segs, n_head_kv)
    for i, seq in enumerate(segs_np):  # the real row counts (the plan reads shapes only)
        for j, (k, _, _) in enumerate(seq):
            a.segs[i * len(seq) + j].n_rows = k.shape[0]
    return kvd.attend_plan(a)


@pytest.mark.parametrize("case", ["unequal_to_4_waves", "unequal_tails_to_4_waves", "seventeen_per_launch"])
def test_planner_paths(oracle, case):
    """Each plan path on the GPU against the oracle, with the plan checked
    first: 16 sequences of 256 ... 8192 rows (8-wave splits would fill 73% of
    the chip, so 4-wave workgroups in 448-row splits); the same with a one-row
    tail segment per sequence (576-row splits); 17 sequences of 4096 rows (two
    launches, splits sized for both)."""
    hq, hkv, d = 40, 8, 128
    rng = np.random.default_rng({"unequal_to_4_waves": 81, "unequal_tails_to_4_waves": 82, "seventeen_per_launch": 83}[case])
    if case == "seventeen_per_launch":
        lens, want = [4096] * 17, (384, 4, 187)
    else:
        lens = [int(n) for n in np.geomspace(256, 8192, 16)]
        want = (448, 4, 94) if case == "unequal_to_4_waves" else (576, 4, 91)
    segs = []
    for n in lens:
        k = inputs.random_kv_rows(rng, n, hkv, d)
        v = inputs.random_kv_rows(rng, n, hkv, d)
        if case == "unequal_tails_to_4_waves":
            segs.append([(k[:n - 1], v[:n - 1], 0), (k[n - 1:], v[n - 1:], n - 1)])
        else:
            segs.append([(k, v, 0)])
    q = inputs.random_q(rng, len(lens), hq, d)
    assert _plan_of(q, segs, hkv) == want
    ref = oracle.attend(q, segs, hkv, d, threads=8)
    check(gpu_attend(q, segs, hkv), ref)


@pytest.mark.parametrize("case", ["4096_lds", "16384_lds", "65536_registers", "batch_registers", "batch_lds", "q4_0_lds"])
def test_load_modes_are_bit_identical(oracle, case):
    """The same call with 16-byte-aligned rows (16-byte loads: straight into
    LDS, or staged in registers at 12 waves per CU) and with rows padded to a
    stride that is not a multiple of 16 (dword loads) gets the same plan, the
    same LDS contents and so bit-identical outputs; both match the oracle."""
    import torch
    from decode_attention_offloaded_amd import kvd
    hq, hkv, d = 40, 8, 128
    rng = np.random.default_rng(sum(map(ord, case)))
    lens = {"4096_lds": [4096], "16384_lds": [16384], "65536_registers": [65536], "q4_0_lds": [4096],
            "batch_registers": [int(n) for n in np.geomspace(256, 8192, 16)], "batch_lds": [2048] * 16}[case]
    v_type = 1 if case == "q4_0_lds" else 0
    vgen = inputs.random_kv_rows_q4_0 if v_type else inputs.random_kv_rows
    segs_np = [[(inputs.random_kv_rows(rng, n, hkv, d), vgen(rng, n, hkv, d), 0)] for n in lens]
    q = inputs.random_q(rng, len(lens), hq, d)

    def run(pad):
        qd = to_dev(q)
        out = torch.full_like(qd, float("nan"))
        segs = []
        for ((k, v, p0),) in segs_np:
            if pad:
                k = np.concatenate([k, np.full((k.shape[0], pad), 0x5A, np.uint8)], axis=1)
                v = np.concatenate([v, np.full((v.shape[0], pad), 0xA5, np.uint8)], axis=1)
            segs.append([(to_dev(k), to_dev(v), p0)])
        kvd.attend_decode(qd, out, segs, hkv, v_type=v_type)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    aligned, padded = run(0), run(8)
    assert np.array_equal(aligned, padded), np.max(np.abs(aligned - padded))
    ref = oracle.attend(q, segs_np, hkv, d, threads=8, v_type=oracle.V_Q4_0 if v_type else oracle.V_Q8_0)
    check(aligned, ref)


@pytest.mark.parametrize("window", [0, 700])
def test_seventeen_sequences_in_two_segments(oracle, window):
    """17 sequences of unequal length, each in two segments: two launches (16
    sequences, then one whose second segment the kernel finds through its
    descriptor), plans sized for both launches, with and without a window;
    every output against the oracle."""
    hq, hkv, d = 40, 8, 128
    rng = np.random.default_rng(1700 + window)
    lens = [int(n) for n in rng.integers(300, 3000, size=17)]
    segs = []
    for n in lens:
        k = inputs.random_kv_rows(rng, n, hkv, d)
        v = inputs.random_kv_rows(rng, n, hkv, d)
        h = n // 3
        segs.append([(k[:h], v[:h], 0), (k[h:], v[h:], h)])
    q = inputs.random_q(rng, len(lens), hq, d)
    ref = oracle.attend(q, segs, hkv, d, window=window, threads=8)
    check(gpu_attend(q, segs, hkv, window=window), ref)
