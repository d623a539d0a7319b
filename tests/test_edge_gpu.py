"""GPU parity on inputs that drive the online softmax to its edges, against
the fp64 oracle at the build's bar (max abs error <= 1e-3).

The running maximum of each split is raised lazily (only when a score passes
it by more than 8 log2 units), the four waves of a workgroup and the splits of
a sequence are merged by their maxima, and tile-streamed partial results are
merged the same way ("F5 -- Advanced KV Cache Techniques", M4 step 6 and W4:
partial attention results merged by their running maxima and sums).  Random
N(0, 1) queries against the standard scales exercise none of that: their
scores spread over about one log2 unit.  These inputs do:
  * one dominant row placed early, late in a split, in a non-first split, in
    the second segment and at the last row;
  * scores that ramp up along the rows, so the maximum is raised many times
    inside one split (each time rescaling what was accumulated);
  * a first stretch of rows more than 200 log2 units below the rest (the
    rescale factor underflows to 0);
  * huge equal scores (binary16 scale 250, codes 127: scores ~ 10^5);
  * the query times 30 (scores spread over more than 100 log2 units);
  * negative and subnormal binary16 K and V scales.
Each goes through the planned call, forced small splits, two segments,
partial results merged by kvd_attend_merge, and q4_0 V where it applies.
"""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from tests.helpers import gpu_attend, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-3
HQ, HKV, D = 40, 8, 128
G = HQ // HKV
NB = D // 32


def check(out, ref, tol=TOL):
    assert np.all(np.isfinite(out)), "non-finite output"
    err = float(np.max(np.abs(out.astype(np.float64) - ref)))
    assert err <= tol, "max abs error %.3g > %.3g" % (err, tol)
    return err


def unpack(rows):
    """uint8 q8_0 rows [n, HKV * NB * 34] -> codes int8 [n, HKV * NB, 32], scale bits uint16 [n, HKV * NB]."""
    b = rows.reshape(rows.shape[0], HKV * NB, 34)
    bits = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
    return b[..., 2:].copy().view(np.int8), bits


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def aligned_codes(q, g):
    """K codes of KV head g that line up with the query of its first query head."""
    v = q[0, g * G].reshape(NB, 32)
    return np.clip(np.rint(127 * v / np.abs(v).max()), -127, 127).astype(np.int8)


def run_all(q, k, v, n, v_type=0, splits=(0, 64, 512), seg_cut=None, parts=3):
    """Attention over rows [0, n) every way the library offers, each against the oracle."""
    import oracle
    import torch
    from decode_attention_offloaded_amd import kvd
    ovt = oracle.V_Q4_0 if v_type else oracle.V_Q8_0
    ref = oracle.attend(q, [[(k, v, 0)]], HKV, D, threads=8, v_type=ovt)
    errs = {}
    for sr in splits:
        out = gpu_attend_vt(q, [[(k, v, 0)]], split_rows=sr, v_type=v_type)
        errs["split%d" % sr] = check(out, ref)
    cut = seg_cut if seg_cut is not None else n // 3
    out = gpu_attend_vt(q, [[(k[:cut], v[:cut], 0), (k[cut:], v[cut:], cut)]], v_type=v_type)
    errs["two_segments"] = check(out, ref)
    # tile-streamed: partial results over row ranges, merged in order
    qd = to_dev(q)
    kd, vd = to_dev(k), to_dev(v)
    edges = [round(i * n / parts) for i in range(parts + 1)]
    pf = kvd.partial_floats(1, HQ, D)
    buf = torch.empty(parts * pf, dtype=torch.float32, device="cuda")
    for i in range(parts):
        a, b = edges[i], edges[i + 1]
        kvd.attend_decode_partial(qd, buf[i * pf:(i + 1) * pf], [[(kd[a:b], vd[a:b], a)]], HKV, q_pos=[n - 1],
                                  v_type=v_type)
    merged = torch.full_like(qd, float("nan"))
    kvd.attend_merge(buf, parts, merged)
    torch.cuda.synchronize()
    errs["partial_merge"] = check(merged.cpu().numpy(), ref)
    return errs


def gpu_attend_vt(q, segs, split_rows=0, v_type=0):
    if v_type == 0:
        return gpu_attend(q, segs, HKV, split_rows=split_rows)
    import torch
    from decode_attention_offloaded_amd import kvd
    qd = to_dev(q)
    out = torch.full_like(qd, float("nan"))
    dsegs = [[(to_dev(kk), to_dev(vv), p0) for (kk, vv, p0) in seq] for seq in segs]
    kvd.attend_decode(qd, out, dsegs, HKV, split_rows=split_rows, v_type=v_type)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("pos", [3, 15, 511, 700, 1500, 2047, 2999])
def test_dominant_row(oracle, pos):
    """Row `pos` of every KV head lines up with its group's first query head at
    a large scale: that head's score there beats the rest by hundreds of
    log2 units (early, at a sub-tile end, at a split end, inside a later
    split, in the second segment of the two-segment call, at the last row)."""
    n = 3000
    rng = np.random.default_rng(100 + pos)
    k = inputs.random_kv_rows(rng, n, HKV, D)
    v = inputs.random_kv_rows(rng, n, HKV, D)
    q = inputs.random_q(rng, 1, HQ, D)
    codes, bits = unpack(k)
    for g in range(HKV):
        codes[pos, g * NB:(g + 1) * NB] = aligned_codes(q, g)
        bits[pos, g * NB:(g + 1) * NB] = f16(0.25)
    k = inputs.pack_q8_0(codes, bits)
    run_all(q, k, v, n, seg_cut=1000)


@pytest.mark.parametrize("v_type", [0, 1])
def test_score_ramp_raises_the_maximum_many_times(oracle, v_type):
    """The K scale of every row grows along the rows, so the aligned score of
    each group's first query head climbs from 0 to ~130 log2 units: the lazy
    maximum is passed by more than 8 about every 150 rows, each time
    rescaling everything accumulated."""
    n = 2500
    rng = np.random.default_rng(7)
    k = inputs.random_kv_rows(rng, n, HKV, D)
    v = inputs.random_kv_rows_q4_0(rng, n, HKV, D) if v_type else inputs.random_kv_rows(rng, n, HKV, D)
    q = inputs.random_q(rng, 1, HQ, D)
    codes, bits = unpack(k)
    ramp = 0.16 * np.arange(n) / n     # K scale 0 .. 0.16
    for g in range(HKV):
        codes[:, g * NB:(g + 1) * NB] = aligned_codes(q, g)
        bits[:, g * NB:(g + 1) * NB] = f16(ramp)[:, None]
    k = inputs.pack_q8_0(codes, bits)
    run_all(q, k, v, n, v_type=v_type)


def test_rescale_factor_underflows(oracle):
    """Rows [0, 1200) score about 227 log2 units below rows [1200, 2000) for
    each group's first query head: the factor that rescales the early
    accumulation, exp2(-227), is 0 in fp32."""
    n = 2000
    rng = np.random.default_rng(8)
    k = inputs.random_kv_rows(rng, n, HKV, D)
    v = inputs.random_kv_rows(rng, n, HKV, D)
    q = inputs.random_q(rng, 1, HQ, D)
    codes, bits = unpack(k)
    for g in range(HKV):
        a = aligned_codes(q, g)
        codes[:1200, g * NB:(g + 1) * NB] = -a
        codes[1200:, g * NB:(g + 1) * NB] = a
        bits[:, g * NB:(g + 1) * NB] = f16(0.15)
    k = inputs.pack_q8_0(codes, bits)
    run_all(q, k, v, n, seg_cut=1100)


@pytest.mark.parametrize("v_type", [0, 1])
def test_huge_equal_scores(oracle, v_type):
    """Every K row is codes 127 at binary16 scale 250 (0x5BD0) and the query is
    all ones: every score is ~3.6e5 and all equal, so the result is the mean
    of V (exp of unshifted scores would overflow)."""
    n = 1500
    rng = np.random.default_rng(9)
    codes = np.full((n, HKV * NB, 32), 127, dtype=np.int8)
    k = inputs.pack_q8_0(codes, np.full((n, HKV * NB), 0x5BD0, dtype=np.uint16))
    v = inputs.random_kv_rows_q4_0(rng, n, HKV, D) if v_type else inputs.random_kv_rows(rng, n, HKV, D)
    q = np.ones((1, HQ, D), dtype=np.float32)
    run_all(q, k, v, n, v_type=v_type)


@pytest.mark.parametrize("v_type", [0, 1])
def test_query_times_30(oracle, v_type):
    """Random K/V and the query times 30: scores spread over more than 100
    log2 units across the rows of every split."""
    n = 4096 + 77
    rng = np.random.default_rng(10)
    k = inputs.random_kv_rows(rng, n, HKV, D)
    v = inputs.random_kv_rows_q4_0(rng, n, HKV, D) if v_type else inputs.random_kv_rows(rng, n, HKV, D)
    q = 30 * inputs.random_q(rng, 1, HQ, D)
    run_all(q, k, v, n, v_type=v_type, splits=(0, 128, 1024))


@pytest.mark.parametrize("v_type", [0, 1])
def test_negative_and_subnormal_scales(oracle, v_type):
    """K and V block scales with random signs, a quarter of them binary16
    subnormals (exponent field 0), the rest normal."""
    n = 1800
    rng = np.random.default_rng(11 + v_type)
    k = inputs.random_kv_rows(rng, n, HKV, D)
    v = inputs.random_kv_rows_q4_0(rng, n, HKV, D) if v_type else inputs.random_kv_rows(rng, n, HKV, D)
    q = 3 * inputs.random_q(rng, 1, HQ, D)

    def scramble(rows, bb):
        blocks = rows.reshape(n, HKV * NB, bb).copy()
        bits = blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << 8)
        sub = rng.random(bits.shape) < 0.25
        bits = np.where(sub, rng.integers(1, 0x400, size=bits.shape, dtype=np.uint16), bits)
        bits = bits | np.where(rng.random(bits.shape) < 0.5, np.uint16(0x8000), np.uint16(0))
        blocks[..., 0] = (bits & 0xFF).astype(np.uint8)
        blocks[..., 1] = (bits >> 8).astype(np.uint8)
        return blocks.reshape(n, -1)

    k = scramble(k, 34)
    v = scramble(v, 18 if v_type else 34)
    # the decoded scales really are subnormal and negative
    kb = k.reshape(n, HKV * NB, 34)
    kbits = kb[..., 0].astype(np.uint16) | (kb[..., 1].astype(np.uint16) << 8)
    assert ((kbits & 0x7C00) == 0).mean() > 0.2 and (kbits >> 15).mean() > 0.4
    run_all(q, k, v, n, v_type=v_type)
