"""kvd_attend_decode_noalloc (split partials in the library's built-in device
array, for callers that cannot allocate) against kvd_attend_decode with a
workspace: the same plan and kernels, so the outputs are bit-identical."""
import ctypes

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

pytestmark = pytest.mark.gpu


def _cache(torch, rng, n, hkv, d, hq, v_type=0):
    k = torch.from_numpy(inputs.random_kv_rows(rng, n, hkv, d)).cuda()
    vg = inputs.random_kv_rows_q4_0 if v_type else inputs.random_kv_rows
    v = torch.from_numpy(vg(rng, n, hkv, d)).cuda()
    q = torch.from_numpy(inputs.random_q(rng, 1, hq, d)).cuda()
    return q, [[(k, v, 0)]]


@pytest.mark.parametrize("v_type", [0, 1])
def test_noalloc_equals_workspace_entry_on_two_calls(v_type):
    """Two calls in a row on one stream, the second smaller (16384 rows, then
    4096 rows, both split, so both use the built-in array), each bit-identical
    to the workspace entry point; device memory in use does not change."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(31 + v_type)
    calls = [_cache(torch, rng, 16384, 8, 128, 40, v_type), _cache(torch, rng, 4096, 8, 128, 40, v_type)]
    refs = []
    for q, segs in calls:
        r = torch.empty_like(q)
        kvd.attend_decode(q, r, segs, 8, workspace=kvd.Workspace(), v_type=v_type)
        refs.append(r)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    outs = [torch.full_like(q, float("nan")) for q, _ in calls]
    warm = torch.empty_like(calls[1][0])
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    with torch.cuda.stream(s):
        # first launches on a new stream may make the HIP runtime set up its own state
        kvd.attend_decode_noalloc(calls[1][0], warm, calls[1][1], 8, stream=s, v_type=v_type)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    print("device memory taken by the first call on a new stream: %d bytes" % (free0 - free1))
    with torch.cuda.stream(s):
        for (q, segs), o in zip(calls, outs):
            kvd.attend_decode_noalloc(q, o, segs, 8, stream=s, v_type=v_type)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free1
    for o, r in zip(outs, refs):
        assert torch.equal(o, r)


def test_noalloc_refuses_calls_beyond_the_array():
    """8 sequences of 16384 rows in 256-row splits: 512 splits x 40 heads x
    130 floats of partials (10.6 MB) exceed the 8 MiB array: KVD_EINVAL, the
    output untouched."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(5)
    k = torch.from_numpy(inputs.random_kv_rows(rng, 16384, 8, 128)).cuda()
    v = torch.from_numpy(inputs.random_kv_rows(rng, 16384, 8, 128)).cuda()
    q = torch.from_numpy(inputs.random_q(rng, 8, 40, 128)).cuda()
    out = torch.full_like(q, 7.0)
    a, keep = kvd.make_args(q, out, [[(k, v, 0)]] * 8, 8, split_rows=256)
    assert kvd.workspace_bytes(a) > 8 << 20
    assert kvd.lib().kvd_attend_decode_noalloc(ctypes.byref(a), None) == kvd.KVD_EINVAL
    assert "scratch" in kvd.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_single_split_and_small_head_dim():
    """Calls without split partials (one split) and head_dim 64: equal to the
    workspace entry point too."""
    import torch
    from decode_attention_offloaded_amd import kvd
    rng = np.random.default_rng(6)
    for n, hkv, d, hq in ((200, 2, 64, 8), (3000, 2, 64, 8), (100, 8, 128, 40)):
        q, segs = _cache(torch, rng, n, hkv, d, hq)
        r = torch.empty_like(q)
        o = torch.full_like(q, float("nan"))
        kvd.attend_decode(q, r, segs, hkv, workspace=kvd.Workspace())
        kvd.attend_decode_noalloc(q, o, segs, hkv)
        torch.cuda.synchronize()
        assert torch.equal(o, r), (n, hkv, d)
