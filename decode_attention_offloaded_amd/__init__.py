"""Decode attention over a q8_0 grouped-query KV cache on MI355X (gfx950),
with the cache in HBM or in pinned host memory delivered one layer ahead.

The library is ``libkvd.so`` (C ABI: ``include/kvd.h``); build it with
``python -m decode_attention_offloaded_amd.build``.  Modules:

- ``kvd``: the ctypes binding (same names as the C ABI; no fallback);
- ``inputs``: seeded synthetic q8_0 / q4_0 rows and queries;
- ``stack``, ``batched``, ``tiled``, ``headsplit``: drivers of the staging
  ring over layer stacks (whole layers, 16 sequences in two residency
  segments, tiles of a layer, a per-head residency split).

Device-resident attention (K and V: uint8 CUDA tensors ``[n_rows, row bytes]``
of q8_0 rows; q and out: float32 ``[n_seq, n_head_q, head_dim]``)::

    from decode_attention_offloaded_amd import kvd
    kvd.attend_decode(q, out, [[(k, v, 0)]], n_head_kv)

Host-resident, one layer ahead (pinned host rows; per layer of a step)::

    ring = kvd.Ring(depth=1, budget_bytes=128 << 20)
    rc, view = ring.stage(l, kvd.STAGE_ACQUIRE, k_ptr, v_ptr, row_bytes, n, n - 1, cap,
                          ordered_k_ptr, ordered_v_ptr, stream=s)
    kvd.attend_decode(q, out, [[(view.k, view.v, view.n_rows, 0, view.row_stride)]], n_head_kv, stream=s)
    ring.release(l, stream=s)
    ring.stage(l + 1, kvd.STAGE_PREFETCH, ...)   # the next layer's stable prefix
"""
