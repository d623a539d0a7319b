"""The C-ABI library loads on a machine without a GPU, exports every entry
point include/kvd.h declares, and rejects invalid arguments before it touches
the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from decode_attention_offloaded_amd import kvd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    with open(os.path.join(ROOT, "include", "kvd.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(kvd_\w+)\s*\(", text, flags=re.M):
        names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kvd_attend_decode", "kvd_ring_create", "kvd_ring_stage_layer", "kvd_ring_release"} <= names
    L = ctypes.CDLL(kvd.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_error_text():
    assert kvd.version().startswith("kvd ")
    assert isinstance(kvd.last_error(), str)


def _args(**kw):
    segs = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, 4096, 0, 1088))
    a = kvd.AttnArgs(1, 40, 8, 128, 1, 0, 0, 0.088, 0x1000, 0x2000, segs, None, None, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a, segs


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("head_dim", 256), ("n_head_q", 41), ("n_head_q", 72),
                                         ("n_seg", 3), ("n_seq", 0), ("window", -1), ("split_rows", 100),
                                         ("q", None), ("out", None), ("reserved", 1)])
def test_attend_rejects_bad_arguments(field, value):
    a, keep = _args(**{field: value})
    assert kvd.lib().kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL
    assert kvd.last_error()


def test_attend_rejects_bad_segments():
    L = kvd.lib()
    for seg in [kvd.KvSeg(0x10000, 0x20000, 4096, 0, 1000),      # stride below the row bytes
                kvd.KvSeg(0x10004, 0x20000, 4096, 0, 1088),      # k not 8-byte aligned (head_dim 128)
                kvd.KvSeg(0x10000, 0x20000, 4096, 0, 1092),      # stride not 8-byte aligned
                kvd.KvSeg(None, 0x20000, 4096, 0, 1088),         # NULL k
                kvd.KvSeg(0x10000, 0x20000, -1, 0, 1088)]:       # negative rows
        a, _ = _args()
        segs = (kvd.KvSeg * 1)(seg)
        a.segs = segs
        assert L.kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL, seg.row_stride


def test_attend_rejects_empty_visible_set():
    a, _ = _args()
    qp = (ctypes.c_int64 * 1)(-5)   # query before every row
    a.q_pos = qp
    assert kvd.lib().kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL
    a.q_pos = None
    a.window = 0
    segs = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, 0, 0, 1088))   # no rows at all
    a.segs = segs
    assert kvd.lib().kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL


def test_workspace_plan():
    a, _ = _args()
    n = kvd.workspace_bytes(a)
    # 4096 rows x 8 KV heads = 512 tiles of 64 rows: one workgroup per CU with
    # two tiles each, i.e. 32 splits per head (split maxima, sums, outputs)
    splits = 32
    expect = 2 * ((splits * 40 * 4 + 255) // 256 * 256) + splits * 40 * 128 * 4
    assert n == expect
    short, _ = _args()
    short.segs = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, 100, 0, 1088))
    assert kvd.workspace_bytes(short) == 0   # a single split writes the output directly
    forced, _ = _args(split_rows=4096)
    assert kvd.workspace_bytes(forced) == 0


def _splits(n_rows_list, seg_rows=None):
    """Total splits the planner makes (kvd_attend_plan), 40 query / 8 KV heads."""
    segs = []
    for n in n_rows_list:
        if seg_rows is None:
            segs.append(kvd.KvSeg(0x10000, 0x20000, n, 0, 1088))
        else:
            h = n // 2
            segs += [kvd.KvSeg(0x10000, 0x20000, h, 0, 1088), kvd.KvSeg(0x10000, 0x20000, n - h, h, 1088)]
    raw = (kvd.KvSeg * len(segs))(*segs)
    a, _ = _args(n_seq=len(n_rows_list), n_seg=1 if seg_rows is None else 2)
    a.segs = raw
    return kvd.attend_plan(a)[2]


@pytest.mark.parametrize("n,splits", [(1024, 16), (2048, 32), (4096, 32), (6144, 32), (8192, 32), (12288, 32),
                                      (16384, 32), (32768, 32), (65536, 32), (131072, 32)])
def test_split_plan_single_sequence(n, splits):
    """Splits per KV head on one sequence of n rows x 8 KV heads on 256 CUs
    (the measured fastest, or within 2% of it): 64-row splits up to 2048 rows,
    128-row ones at 4096 rows (4-wave workgroups, one per CU), then one 8- or
    12-wave workgroup per CU, 32 splits per head."""
    assert _splits([n]) == splits


@pytest.mark.parametrize("n,split_rows,waves", [(256, 64, 4), (4096, 128, 4), (6144, 192, 8), (8192, 256, 8),
                                                 (16384, 512, 8), (49152, 1536, 12), (131072, 4096, 12)])
def test_planned_waves(n, split_rows, waves):
    """Rows per split and waves per decode workgroup on 256 CUs, one sequence
    of n rows x 8 KV heads: 4-wave workgroups below 12 sub-tiles of 16 rows
    per CU, 8-wave ones below 96, then 12-wave ones (one per CU)."""
    a, _ = _args()
    a.segs = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, n, 0, 1088))
    sr, w, total = kvd.attend_plan(a)
    assert (sr, w) == (split_rows, waves)
    assert total == -(-n // sr)
    bad, _ = _args()
    bad.head_dim = 96
    assert kvd.lib().kvd_attend_plan(ctypes.byref(bad), None, None, None) == kvd.KVD_EINVAL
    assert kvd.lib().kvd_attend_plan(ctypes.byref(a), None, None, None) == kvd.KVD_OK


@pytest.mark.parametrize("d,n_head_kv,n,split_rows,waves", [
    (128, 8, 64, 64, 4), (128, 8, 128, 128, 4), (128, 8, 129, 192, 8), (128, 8, 192, 192, 8), (128, 8, 193, 64, 4),
    (64, 2, 128, 128, 4), (64, 2, 256, 256, 8), (64, 2, 384, 384, 8), (64, 2, 385, 64, 4), (64, 8, 320, 320, 8)])
def test_short_context_plan(d, n_head_kv, n, split_rows, waves):
    """Short contexts with at most one workgroup per CU: one split (no combine
    launch) up to 12 sub-tiles (16 rows at head_dim 128, 32 at 64), as one
    8-wave workgroup beyond 128 rows; longer ones are split as usual."""
    a, _ = _args()
    a.head_dim = d
    a.n_head_kv = n_head_kv
    a.n_head_q = n_head_kv * 4
    a.segs = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, n, 0, n_head_kv * d // 32 * 34))
    sr, w, total = kvd.attend_plan(a)
    assert (sr, w, total) == (split_rows, waves, -(-n // split_rows))


def test_short_context_batch_plan():
    """Workgroups outnumbering the CUs (64 sequences x 8 KV heads of 250 rows):
    one split per sequence up to 256 rows, waves from the work per CU."""
    segs = (kvd.KvSeg * 64)(*[kvd.KvSeg(0x10000, 0x20000, 250, 0, 1088) for _ in range(64)])
    a, _ = _args(n_seq=64)
    a.segs = segs
    assert kvd.attend_plan(a) == (256, 8, 64)


def _plan_of(seg_lists):
    """kvd_attend_plan for sequences given as lists of (n_rows, pos0), 40 query / 8 KV heads."""
    segs = [kvd.KvSeg(0x10000, 0x20000, n, p0, 1088) for sl in seg_lists for n, p0 in sl]
    a, _ = _args(n_seq=len(seg_lists), n_seg=len(seg_lists[0]))
    a.segs = (kvd.KvSeg * len(segs))(*segs)
    return kvd.attend_plan(a)


def test_split_plan_batch():
    """16 sequences of unequal length in two segments each (80231 rows): 12-wave
    workgroups in 1664-row splits would fill 75% of the chip's time (two
    rounds, many short last splits), so the plan takes 4-wave workgroups in
    1024-row splits, 92 in all, about three per CU."""
    lens = [1024, 1024, 1862, 1990, 2813, 3712, 3769, 4264, 5376, 5801, 6363, 6588, 7292, 8678, 9634, 10041]
    assert _splits(lens, seg_rows=True) == sum(-(-(n // 2) // 1024) + -(-(n - n // 2) // 1024) for n in lens) == 92
    assert _plan_of([[(n // 2, 0), (n - n // 2, n // 2)] for n in lens]) == (1024, 4, 92)


@pytest.mark.parametrize("seg_lists,plan", [
    ([[(4096, 0)]] * 16, (2048, 12, 32)),                              # equal: fills the chip
    ([[(16383, 0), (1, 16383)]] * 4, (2368, 12, 32)),                 # equal, each with a one-row tail
    ([[(131072, 0)], [(65536, 0)]], (6272, 12, 32)),                  # unequal but long: 98% filled
    ([[(8192, 0)]] * 8 + [[(2048, 0)]] * 8, (2752, 12, 32)),          # two lengths: 93% filled
    ([[(n, 0)] for n in (256, 322, 406, 512, 645, 812, 1024, 1290, 1625, 2048, 2580, 3250, 4096, 5160, 6501, 8192)],
     (448, 4, 94)),                                                    # 256 ... 8192 rows: 73% -> 4 waves
])
def test_plan_fill_rule(seg_lists, plan):
    """8- and 12-wave workgroups are kept where their splits fill at least 85%
    of the chip's time (visible rows x KV heads over CUs x split rows x
    rounds); below that, sequences of unequal length go to 4-wave workgroups
    in their own splits.  Single sequences always keep the 8/12-wave plan."""
    assert _plan_of(seg_lists) == plan


@pytest.mark.parametrize("seg_lists,stride,mode", [
    ([[(4096, 0)]], 1088, 2),            # 4 waves, one workgroup per CU: straight into LDS
    ([[(16384, 0)]], 1088, 2),           # 8 waves
    ([[(131072, 0)]], 1088, 1),          # 12 waves: staged in registers
    ([[(n, 0)] for n in (256, 322, 406, 512, 645, 812, 1024, 1290, 1625, 2048, 2580, 3250, 4096, 5160, 6501, 8192)],
     1088, 1),                           # 4 waves, about three per CU
    ([[(4096, 0)]], 1096, 0),            # a row stride that is not a multiple of 16: dword loads
])
def test_load_mode(seg_lists, stride, mode):
    """kvd_attend_load_mode: the decode kernel's load mode for the call's first
    launch, from the plan and the alignment of the K/V pointers and strides
    (256 CUs)."""
    segs = [kvd.KvSeg(0x10000, 0x20000, n, p0, stride) for sl in seg_lists for n, p0 in sl]
    a, _ = _args(n_seq=len(seg_lists), n_seg=len(seg_lists[0]))
    a.segs = (kvd.KvSeg * len(segs))(*segs)
    assert kvd.attend_load_mode(a) == mode
    assert kvd.lib().kvd_attend_load_mode(ctypes.byref(a), None) == kvd.KVD_EINVAL


@pytest.mark.parametrize("n_seq,n,plan", [(16, 4096, (2048, 12, 32)), (17, 4096, (384, 4, 187)),
                                          (32, 4096, (2048, 12, 64)), (64, 4096, (2048, 12, 128)),
                                          (64, 1024, (512, 8, 128))])
def test_plan_per_launch_capacity(n_seq, n, plan):
    """A call of more than 16 sequences runs as consecutive launches of up to
    16, so splits and waves are chosen for the CUs of all its launches: each
    launch of 16 sequences of 4096 rows gets 2048-row splits (256 workgroups),
    not one 4096-row split (128, half the chip)."""
    assert _plan_of([[(n, 0)]] * n_seq) == plan


def test_workspace_too_small_is_rejected():
    a, _ = _args()
    a.workspace = 0x100000
    a.workspace_bytes = 1024
    assert kvd.lib().kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL


def test_ring_create_and_stats_without_device_work():
    L = kvd.lib()
    assert not L.kvd_ring_create(-1, 1 << 20)
    assert not L.kvd_ring_create(65, 1 << 20)
    r = kvd.Ring(1, 128 << 20)
    st = r.stats()
    assert (st["depth"], st["n_slots"], st["engaged"], st["declined"], st["ring_bytes"]) == (1, 3, 0, 0, 0)
    small = kvd.RingStats()
    assert L.kvd_ring_stats_get(r._h, ctypes.byref(small), 8) == kvd.KVD_EINVAL
    # argument checks come before any HIP call
    with pytest.raises(kvd.KvdError) as e:
        r.stage(0, kvd.STAGE_ACQUIRE, 0x1000, 0x2000, 1088, 10, 9, 5, stream=0)  # n_rows > cap_rows
    assert e.value.code == kvd.KVD_EINVAL
    with pytest.raises(kvd.KvdError):
        r.stage(0, 7, 0x1000, 0x2000, 1088, 10, 9, 10, stream=0)  # bad flags
    with pytest.raises(kvd.KvdError):
        r.stage(0, kvd.STAGE_PREFETCH, 0x1000, 0x2000, 1088, 10, 11, 10, stream=0)  # stable > n_rows
    # the test-support transfer delay: validated, no device work
    r.set_transfer_delay(100, 7)
    r.set_transfer_delay(0)
    assert L.kvd_ring_set_transfer_delay(r._h, 100001, 1) == kvd.KVD_EINVAL
    assert L.kvd_ring_set_transfer_delay(None, 10, 1) == kvd.KVD_EINVAL
    r.close()
    L.kvd_ring_destroy(None)


def test_tile_rows_is_the_largest_fitting_multiple_of_64(oracle):
    """kvd_ring_tile_rows against a brute-force search with the oracle's ring sizing."""
    rb = 1088
    for depth in (1, 2, 3):
        for budget in (0, 1 << 20, 64 << 20, 128 << 20, 134_111_232, 134_111_231, 1 << 30):
            rc, rows = kvd.tile_rows(depth, budget, rb)
            best = 0
            r = 64
            while oracle.ring_fits(depth, r, rb, budget):
                best = r
                r += 64
            if best == 0:
                assert rc == kvd.KVD_DECLINED and rows == 0, (depth, budget)
            else:
                assert rc == kvd.KVD_OK and rows == best, (depth, budget, rows, best)
    # 128 MiB at depth 1: 20544 rows (3 slots x 2 x 20544 x 1088 = 134,111,232 B)
    assert kvd.tile_rows(1, 128 << 20, rb) == (kvd.KVD_OK, 20544)
    # the compute-window bound: one tile's K+V at most max_tile_bytes
    rc, rows = kvd.tile_rows(1, 1 << 30, rb, max_tile_bytes=2.7e6)
    assert rc == kvd.KVD_OK and rows == int(2.7e6 / (2 * rb)) // 64 * 64
    for bad in ((0, 1 << 20, rb, 0.0), (1, 1 << 20, 0, 0.0), (1, 1 << 20, rb, -1.0), (1, 1 << 20, rb, float("nan"))):
        with pytest.raises(kvd.KvdError):
            kvd.tile_rows(*bad)


def test_merge_and_partial_validate_before_launch():
    L = kvd.lib()
    assert L.kvd_attend_merge(None, 1, 1, 8, 128, ctypes.c_void_p(0x1000), None) == kvd.KVD_EINVAL
    assert L.kvd_attend_merge(ctypes.c_void_p(0x1000), 0, 1, 8, 128, ctypes.c_void_p(0x2000), None) == kvd.KVD_EINVAL
    assert L.kvd_attend_merge(ctypes.c_void_p(0x1000), 2, 1, 8, 96, ctypes.c_void_p(0x2000), None) == kvd.KVD_EINVAL
    assert L.kvd_attend_merge(ctypes.c_void_p(0x1008), 2, 1, 8, 128, ctypes.c_void_p(0x2000), None) == kvd.KVD_EINVAL
    assert L.kvd_attend_merge(ctypes.c_void_p(0x1000), 2, 1, 7, 128, ctypes.c_void_p(0x2000), None) == kvd.KVD_EINVAL
    a, _ = _args()
    assert L.kvd_attend_decode_partial(ctypes.byref(a), None, None) == kvd.KVD_EINVAL
    assert L.kvd_attend_decode_partial(ctypes.byref(a), ctypes.c_void_p(0x1004), None) == kvd.KVD_EINVAL


def test_v_type_and_v_stride_are_validated():
    L = kvd.lib()
    a, keep = _args()
    a.v_type = 7
    assert L.kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL
    # q4_0 V rows are 8 x 4 x 18 = 576 bytes: a V stride below that is rejected
    segs = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, 4096, 0, 1088, 572))
    a, _ = _args(segs=segs, v_type=kvd.TYPE_Q4_0)
    assert L.kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL
    # q8_0 V with a V stride below the q8_0 row
    segs2 = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, 4096, 0, 1088, 1000))
    a, _ = _args(segs=segs2)
    assert L.kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL
    # misaligned q4_0 V base
    segs3 = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20002, 4096, 0, 1088, 576))
    a, _ = _args(segs=segs3, v_type=kvd.TYPE_Q4_0)
    assert L.kvd_attend_decode(ctypes.byref(a), None) == kvd.KVD_EINVAL
    # a valid q4_0 geometry plans (workspace size is independent of the V type)
    segs4 = (kvd.KvSeg * 1)(kvd.KvSeg(0x10000, 0x20000, 4096, 0, 1088, 576))
    a4, _ = _args(segs=segs4, v_type=kvd.TYPE_Q4_0)
    a8, _ = _args()
    assert kvd.workspace_bytes(a4) == kvd.workspace_bytes(a8)


def test_link_probe_validates_before_touching_the_gpu():
    L = kvd.lib()
    g = ctypes.c_double(0.0)
    for args in ((100, 2, 10), (1 << 20, 0, 10), (1 << 20, 5, 10), (1 << 20, 2, 0), ((9 << 30), 1, 1)):
        assert L.kvd_link_probe(args[0], args[1], args[2], ctypes.byref(g)) == kvd.KVD_EINVAL, args
    assert L.kvd_link_probe(1 << 20, 2, 10, None) == kvd.KVD_EINVAL


def test_hbm_read_probe_validates_before_touching_the_gpu():
    L = kvd.lib()
    g = ctypes.c_double(0.0)
    for args in ((100, 3), ((1 << 20) + 8, 3), ((1 << 20) - 16, 3), ((65 << 30), 3), (1 << 20, 0), (1 << 20, 1001)):
        assert L.kvd_hbm_read_probe(args[0], args[1], ctypes.byref(g)) == kvd.KVD_EINVAL, args
    assert L.kvd_hbm_read_probe(1 << 20, 3, None) == kvd.KVD_EINVAL
