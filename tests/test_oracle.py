"""Pins for the fp64 oracle: things the pages and the mathematics fix, chosen so
that a plausible mistake in the oracle (a dropped term, a wrong sign or index,
swapped K/V, a wrong head mapping, a missing max subtraction, a wrong decode of
the binary16 scale) fails at least one of them.  None of these re-types the
oracle's formula: they use closed forms, invariants, exhaustive comparison with
numpy's binary16, hand-decoded golden blocks and a pure-Python brute force.
"""
import math
import os

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def one_block_rows(codes_per_row, scale_bits_per_row, n_head_kv=1, head_dim=32):
    """Rows of a cache with explicit codes int8 [n, n_blocks, 32] and scales uint16 [n, n_blocks]."""
    codes = np.asarray(codes_per_row, dtype=np.int8)
    bits = np.asarray(scale_bits_per_row, dtype=np.uint16)
    return inputs.pack_q8_0(codes, bits)


def f16bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- binary16 / q8_0

def test_f16_decode_exhaustive(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def _golden_blocks():
    cases = []
    with open(os.path.join(GOLDEN, "q8_0_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            assert parts[0] == "case"
            bits = int(parts[1], 16)
            pairs = []
            for p in parts[2:]:
                pos, rest = p.split(":")
                code, val = rest.split("=")
                pairs.append((int(pos), int(code), float(val)))
            cases.append((bits, pairs))
    return cases


@pytest.mark.parametrize("case", _golden_blocks())
def test_dequant_golden_blocks(oracle, case):
    bits, pairs = case
    codes = np.zeros((1, 32), dtype=np.int8)
    for pos, code, _ in pairs:
        codes[0, pos] = code
    blk = inputs.pack_q8_0(codes, np.array([bits], dtype=np.uint16))
    assert blk.shape == (34,)
    vals = oracle.dequant_q8_0(blk)
    expect = np.zeros(32)
    for pos, _, val in pairs:
        expect[pos] = val
    assert np.array_equal(vals, expect)


def test_pack_layout_byte_offsets():
    """Scale little-endian at byte 0, codes at bytes 2..33, blocks back to back."""
    codes = np.arange(-32, 32, dtype=np.int8).reshape(2, 32)
    bits = np.array([0x1234, 0xABCD], dtype=np.uint16)
    b = inputs.pack_q8_0(codes, bits)
    assert b.shape == (68,)
    assert (b[0], b[1], b[34], b[35]) == (0x34, 0x12, 0xCD, 0xAB)
    assert np.array_equal(b[2:34].view(np.int8), codes[0])
    assert np.array_equal(b[36:68].view(np.int8), codes[1])
    assert inputs.row_bytes(8, 128) == 1088 and inputs.row_bytes(2, 64) == 136


# ---------------------------------------------------------------- attention closed forms

def _rand_cache(seed, n, n_head_kv, head_dim):
    rng = np.random.default_rng(seed)
    k = inputs.random_kv_rows(rng, n, n_head_kv, head_dim)
    v = inputs.random_kv_rows(rng, n, n_head_kv, head_dim)
    return rng, k, v


def _v_values(oracle, v_rows, n_head_kv, head_dim):
    """Dequantised V as [n, n_head_kv, head_dim] through the (separately pinned) decoder."""
    n = v_rows.shape[0]
    return oracle.dequant_q8_0(v_rows).reshape(n, n_head_kv, head_dim)


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (40, 8, 128), (4, 4, 32)])
def test_one_token_context_returns_v(oracle, hq, hkv, d):
    rng, k, v = _rand_cache(1, 1, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    vv = _v_values(oracle, v, hkv, d)[0]
    g = np.arange(hq) // (hq // hkv)
    assert np.array_equal(out[0], vv[g])


def test_all_equal_keys_give_mean_of_v(oracle):
    hq, hkv, d, n = 8, 2, 64, 37
    rng, k, v = _rand_cache(2, n, hkv, d)
    k[:] = k[0]
    q = inputs.random_q(rng, 1, hq, d)
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    mean = _v_values(oracle, v, hkv, d).mean(axis=0)
    g = np.arange(hq) // (hq // hkv)
    np.testing.assert_allclose(out[0], mean[g], rtol=0, atol=1e-13)


def test_zero_query_gives_mean_of_v(oracle):
    hq, hkv, d, n = 6, 3, 64, 50
    rng, k, v = _rand_cache(3, n, hkv, d)
    q = np.zeros((1, hq, d), dtype=np.float32)
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    mean = _v_values(oracle, v, hkv, d).mean(axis=0)
    g = np.arange(hq) // (hq // hkv)
    np.testing.assert_allclose(out[0], mean[g], rtol=0, atol=1e-13)


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 32), (6, 3, 64), (4, 4, 32), (8, 1, 64), (40, 8, 128)])
def test_gqa_mapping_brute_force(oracle, hq, hkv, d):
    """Every V value of KV head g is g + 1 (scale 1.0, code g + 1); query head h
    must then return floor(h / G) + 1.  An interleaved h mod n_head_kv mapping fails."""
    n = 7
    rng, k, _ = _rand_cache(4, n, hkv, d)
    nb = d // 32
    codes = np.zeros((n, hkv * nb, 32), dtype=np.int8)
    for g in range(hkv):
        codes[:, g * nb:(g + 1) * nb, :] = g + 1
    v = inputs.pack_q8_0(codes, np.full((n, hkv * nb), 0x3C00, dtype=np.uint16))
    q = inputs.random_q(rng, 1, hq, d)
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    G = hq // hkv
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], h // G + 1, rtol=0, atol=1e-12)


def test_two_row_closed_form(oracle):
    """Two rows, head_dim 32, q = 1: row 0 has K codes 0 (score 0), row 1 has K
    codes 1 at scale 1 (q.k = 32).  With scale = ln(3)/32 the score gap is ln 3,
    so the weights are 1/4 and 3/4; V rows are 4 and 8 -> 0.25*4 + 0.75*8 = 7.
    With q = -1 the gap flips: 0.75*4 + 0.25*8 = 5.  Swapping K and V, dropping
    the scale, or flipping the sign of the exponent all change these numbers."""
    one = 0x3C00
    k = one_block_rows([[[0] * 32], [[1] * 32]], [[one], [one]])
    v = one_block_rows([[[4] * 32], [[8] * 32]], [[one], [one]])
    scale = math.log(3.0) / 32.0
    out = oracle.attend(np.ones((1, 1, 32), np.float32), [[(k, v, 0)]], 1, 32, scale=scale)
    np.testing.assert_allclose(out[0, 0], 7.0, rtol=0, atol=1e-12)
    out = oracle.attend(-np.ones((1, 1, 32), np.float32), [[(k, v, 0)]], 1, 32, scale=scale)
    np.testing.assert_allclose(out[0, 0], 5.0, rtol=0, atol=1e-12)


def test_k_scale_enters_the_score(oracle):
    """Same as the two-row case but row 1's K scale is 0.5 with codes 2: the
    product d * code is still 1, so the result must still be 7."""
    one, half = 0x3C00, 0x3800
    k = one_block_rows([[[0] * 32], [[2] * 32]], [[one], [half]])
    v = one_block_rows([[[4] * 32], [[8] * 32]], [[one], [one]])
    out = oracle.attend(np.ones((1, 1, 32), np.float32), [[(k, v, 0)]], 1, 32,
                        scale=math.log(3.0) / 32.0)
    np.testing.assert_allclose(out[0, 0], 7.0, rtol=0, atol=1e-12)


def test_default_scale_is_inverse_sqrt_head_dim(oracle):
    """q = 1, row 1 codes 1: q.k = 64 at head_dim 64, so with 1/sqrt(64) the gap is 8."""
    one = 0x3C00
    k = one_block_rows([[[0] * 32] * 2, [[1] * 32] * 2], [[one] * 2, [one] * 2])
    v = one_block_rows([[[0] * 32] * 2, [[1] * 32] * 2], [[one] * 2, [one] * 2])
    out = oracle.attend(np.ones((1, 1, 64), np.float32), [[(k, v, 0)]], 1, 64)
    w1 = math.exp(8.0) / (1.0 + math.exp(8.0))
    np.testing.assert_allclose(out[0, 0], w1, rtol=1e-14)


def test_dominant_row(oracle):
    """A row whose score beats every other by >= 60 owns the output (e^-60 ~ 1e-26)."""
    hq, hkv, d, n = 1, 1, 32, 9
    rng, k, v = _rand_cache(5, n, hkv, d)
    k[:] = one_block_rows([[[0] * 32]] * n, [[0x3C00]] * n)
    k[4] = one_block_rows([[[127] * 32]], [[0x3C00]])[0]
    q = np.full((1, 1, 32), 1.0, np.float32)  # score of row 4: 127*32/sqrt(32) ~ 718
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    np.testing.assert_allclose(out[0, 0], _v_values(oracle, v, 1, 32)[4, 0], rtol=1e-15)


def test_huge_equal_scores_do_not_overflow(oracle):
    """Scores of ~ +-5000 overflow exp() unless the maximum is subtracted."""
    n = 5
    k = one_block_rows([[[127] * 32]] * n, [[0x5BD0]] * n)  # scale 250
    rng, _, v = _rand_cache(6, n, 1, 32)
    q = np.full((1, 1, 32), 1.0, np.float32)
    out = oracle.attend(q, [[(k, v, 0)]], 1, 32)
    np.testing.assert_allclose(out[0, 0], _v_values(oracle, v, 1, 32).mean(axis=0)[0], atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_permuting_rows_leaves_output_unchanged(oracle):
    hq, hkv, d, n = 8, 2, 64, 40
    rng, k, v = _rand_cache(7, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    perm = rng.permutation(n)
    a = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    b = oracle.attend(q, [[(k[perm], v[perm], 0)]], hkv, d)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_output_inside_convex_hull_of_v(oracle):
    hq, hkv, d, n = 8, 2, 64, 33
    rng, k, v = _rand_cache(8, n, hkv, d)
    q = 3 * inputs.random_q(rng, 1, hq, d)
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)[0]
    vv = _v_values(oracle, v, hkv, d)
    G = hq // hkv
    for h in range(hq):
        lo = vv[:, h // G].min(axis=0)
        hi = vv[:, h // G].max(axis=0)
        assert np.all(out[h] >= lo - 1e-12) and np.all(out[h] <= hi + 1e-12)


def test_two_segments_equal_one(oracle):
    """Rows split into an older (host) and a newer (device) segment give the
    same result as one segment: softmax over the union of rows."""
    hq, hkv, d, n = 8, 2, 64, 29
    rng, k, v = _rand_cache(9, n, hkv, d)
    q = inputs.random_q(rng, 2, hq, d)
    cut = 11
    one = oracle.attend(q, [[(k, v, 0)]] * 2, hkv, d)
    two = oracle.attend(q, [[(k[:cut], v[:cut], 0), (k[cut:], v[cut:], cut)]] * 2, hkv, d)
    np.testing.assert_allclose(one, two, rtol=0, atol=1e-14)


def test_row_stride_padding_is_ignored(oracle):
    hq, hkv, d, n = 8, 2, 64, 12
    rng, k, v = _rand_cache(10, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    pad = 40
    kp = np.concatenate([k, rng.integers(0, 256, (n, pad), dtype=np.uint8)], axis=1)
    vp = np.concatenate([v, rng.integers(0, 256, (n, pad), dtype=np.uint8)], axis=1)
    a = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    b = oracle.attend(q, [[(kp, vp, 0)]], hkv, d)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- the symmetric entry point

@pytest.mark.parametrize("pad", [0, 24])
def test_symmetric_entry_one_row_and_gqa(oracle, pad):
    """kvd_oracle_attend_f64 (q8_0 K and V, one row stride) on its own: a
    one-row context returns that row's V for every query head of the group, and
    with every V value of KV head g equal to g + 1 query head h returns
    floor(h / G) + 1 (also through padded rows)."""
    hq, hkv, d = 8, 2, 64
    rng, k, v = _rand_cache(40 + pad, 1, hkv, d)
    if pad:
        k = np.concatenate([k, rng.integers(0, 256, (1, pad), dtype=np.uint8)], axis=1)
        v = np.concatenate([v, rng.integers(0, 256, (1, pad), dtype=np.uint8)], axis=1)
    q = inputs.random_q(rng, 1, hq, d)
    out = oracle.attend_symmetric(q, [[(k, v, 0)]], hkv, d)
    vv = _v_values(oracle, v[:, :inputs.row_bytes(hkv, d)], hkv, d)[0]
    assert np.array_equal(out[0], vv[np.arange(hq) // (hq // hkv)])
    n, nb = 6, d // 32
    _, k, _ = _rand_cache(41 + pad, n, hkv, d)
    codes = np.zeros((n, hkv * nb, 32), dtype=np.int8)
    for g in range(hkv):
        codes[:, g * nb:(g + 1) * nb, :] = g + 1
    v = inputs.pack_q8_0(codes, np.full((n, hkv * nb), 0x3C00, dtype=np.uint16))
    if pad:
        k = np.concatenate([k, rng.integers(0, 256, (n, pad), dtype=np.uint8)], axis=1)
        v = np.concatenate([v, rng.integers(0, 256, (n, pad), dtype=np.uint8)], axis=1)
    out = oracle.attend_symmetric(q, [[(k, v, 0)]], hkv, d)
    np.testing.assert_allclose(out[0], (np.arange(hq) // (hq // hkv) + 1)[:, None] + 0 * out[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_seg,window,pad", [(1, 0, 0), (1, 0, 40), (2, 0, 40), (2, 7, 40), (1, 9, 24), (2, 0, 0)])
def test_symmetric_entry_equals_the_general_entry(oracle, n_seg, window, pad):
    """kvd_oracle_attend_f64 passes each segment's single row stride to the
    pinned general entry point as both the K and the V stride: on padded q8_0
    rows, in one or two segments, with and without a window, the two agree bit
    for bit (a wrong stride copy in the adapter reads the padding)."""
    hq, hkv, d, n = 8, 2, 64, 23
    rng, k, v = _rand_cache(50 + pad + window + n_seg, n, hkv, d)
    if pad:
        k = np.concatenate([k, rng.integers(0, 256, (n, pad), dtype=np.uint8)], axis=1)
        v = np.concatenate([v, rng.integers(0, 256, (n, pad), dtype=np.uint8)], axis=1)
    q = inputs.random_q(rng, 2, hq, d)
    if n_seg == 1:
        segs = [[(k, v, 3)], [(k[:15], v[:15], 0)]]
    else:
        segs = [[(k[:9], v[:9], 0), (k[9:], v[9:], 9)], [(k[:4], v[:4], 10), (k[4:15], v[4:15], 14)]]
    a = oracle.attend_symmetric(q, segs, hkv, d, window=window)
    b = oracle.attend(q, segs, hkv, d, window=window)
    assert np.array_equal(a, b)
    # and the padding really is skipped: the unpadded rows give the same bytes
    rb = inputs.row_bytes(hkv, d)
    bare = [[(kk[:, :rb], vv[:, :rb], p0) for (kk, vv, p0) in seq] for seq in segs]
    assert np.array_equal(a, oracle.attend(q, bare, hkv, d, window=window))


# ---------------------------------------------------------------- masks

def test_window_one_returns_newest_v(oracle):
    hq, hkv, d, n = 8, 2, 64, 20
    rng, k, v = _rand_cache(11, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    out = oracle.attend(q, [[(k, v, 100)]], hkv, d, window=1)
    vv = _v_values(oracle, v, hkv, d)[-1]
    assert np.array_equal(out[0], vv[np.arange(hq) // 4])


def test_window_at_least_context_is_full_attention(oracle):
    hq, hkv, d, n = 8, 2, 64, 20
    rng, k, v = _rand_cache(12, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    full = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    for w in (n, n + 1, 10**6):
        assert np.array_equal(full, oracle.attend(q, [[(k, v, 0)]], hkv, d, window=w))


def test_window_keeps_exactly_the_last_w_rows(oracle):
    hq, hkv, d, n, w = 8, 2, 64, 30, 9
    rng, k, v = _rand_cache(13, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    a = oracle.attend(q, [[(k, v, 0)]], hkv, d, window=w)
    b = oracle.attend(q, [[(k[n - w:], v[n - w:], n - w)]], hkv, d)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_query_position_is_causal(oracle):
    hq, hkv, d, n = 8, 2, 64, 30
    rng, k, v = _rand_cache(14, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    a = oracle.attend(q, [[(k, v, 0)]], hkv, d, q_pos=[17])
    b = oracle.attend(q, [[(k[:18], v[:18], 0)]], hkv, d)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_empty_visible_set_is_rejected(oracle):
    rng, k, v = _rand_cache(15, 4, 1, 32)
    q = inputs.random_q(rng, 1, 1, 32)
    with pytest.raises(ValueError):
        oracle.attend(q, [[(k, v, 10)]], 1, 32, q_pos=[5])


# ---------------------------------------------------------------- brute force

def _brute_force(q, k_rows, v_rows, hkv, d, scale):
    """Pure-Python decode of every block from its bytes and a literal softmax.
    Tiny inputs only.  Independent of the C code (own binary16 decode via struct)."""
    import struct
    n = k_rows.shape[0]
    nb = d // 32

    def val(row, g, i):
        off = (g * nb + i // 32) * 34
        dd = struct.unpack("<e", bytes(row[off:off + 2]))[0]
        c = struct.unpack("b", bytes(row[off + 2 + i % 32:off + 3 + i % 32]))[0]
        return dd * c

    hq = q.shape[0]
    G = hq // hkv
    out = []
    for h in range(hq):
        g = h // G
        s = [scale * math.fsum(float(q[h, i]) * val(k_rows[t], g, i) for i in range(d)) for t in range(n)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        den = math.fsum(w)
        out.append([math.fsum(w[t] * val(v_rows[t], g, i) for t in range(n)) / den for i in range(d)])
    return np.array(out)


@pytest.mark.parametrize("hq,hkv,d,n", [(2, 1, 32, 3), (4, 2, 64, 5), (6, 3, 32, 4)])
def test_brute_force_tiny(oracle, hq, hkv, d, n):
    rng, k, v = _rand_cache(16 + n, n, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    ref = _brute_force(q[0], k, v, hkv, d, 1 / math.sqrt(d))
    out = oracle.attend(q, [[(k, v, 0)]], hkv, d)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- ring sizing (pages' table)

def _ring_table():
    rows = []
    with open(os.path.join(GOLDEN, "ring_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(tuple(int(x) for x in line.split()))
    return rows


def test_ring_bytes_reproduce_printed_ring_column(oracle):
    for ctx, delta_mib, ring_col in _ring_table():
        b = oracle.ring_bytes(1, ctx, 1088)
        assert abs(b / 1e6 - ring_col) < 1.0, (ctx, b)
        mib = b / 2**20
        assert 0.0 < delta_mib - mib < 3.0, (ctx, delta_mib, mib)
        # the page sizes the 128k ring at roughly three layers' K+V: exactly three at depth 1
        assert b == 3 * ctx * 2176


def test_ring_budget_decisions_match_the_page(oracle):
    MiB = 2**20
    # default 128 MiB: 4k and 16k pipeline, 32k declines (device memory identical to ordered)
    assert oracle.ring_fits(1, 4096, 1088, 128 * MiB)
    assert oracle.ring_fits(1, 16384, 1088, 128 * MiB)
    assert not oracle.ring_fits(1, 32768, 1088, 128 * MiB)
    # a 512 MiB budget buys the 32k ring (206 MiB)
    assert oracle.ring_fits(1, 32768, 1088, 512 * MiB)
    # the table's run: 128k fits, 262k declines; 1 GiB is such a budget
    assert oracle.ring_fits(1, 131072, 1088, 1024 * MiB)
    assert not oracle.ring_fits(1, 262144, 1088, 1024 * MiB)
    # depth 0 is the ordered path: no ring at all
    assert oracle.ring_bytes(0, 16384, 1088) == 0 and not oracle.ring_fits(0, 16384, 1088, 1 << 40)
    # the 128k sweep: depth 2 needs 1088 MiB, over 1 GiB
    assert oracle.ring_bytes(2, 131072, 1088) == 1088 * MiB
    assert not oracle.ring_fits(2, 131072, 1088, 1024 * MiB)
    # inclusive comparison
    assert oracle.ring_fits(1, 16384, 1088, oracle.ring_bytes(1, 16384, 1088))
