"""Shared helpers for the test suite: synthetic caches (from the seeded input
module) and small adapters between numpy, torch and the oracle."""
from __future__ import annotations

import numpy as np

from decode_attention_offloaded_amd import inputs


def make_cache(seed, n_rows, n_head_kv, head_dim, pad=0):
    """K and V rows as uint8 [n_rows, row_bytes + pad] (pad bytes are random junk)."""
    rng = np.random.default_rng(seed)
    k = inputs.random_kv_rows(rng, n_rows, n_head_kv, head_dim)
    v = inputs.random_kv_rows(rng, n_rows, n_head_kv, head_dim)
    if pad:
        k = np.concatenate([k, rng.integers(0, 256, (n_rows, pad), dtype=np.uint8)], axis=1)
        v = np.concatenate([v, rng.integers(0, 256, (n_rows, pad), dtype=np.uint8)], axis=1)
    return rng, k, v


def head_slice(rows: np.ndarray, g: int, n_head_kv: int, head_dim: int) -> np.ndarray:
    """Bytes of KV head g from every row -> a one-KV-head cache (for sampled checks)."""
    cb = head_dim // 32 * 34
    return np.ascontiguousarray(rows[:, g * cb:(g + 1) * cb])


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_attend(q, segs_np, n_head_kv, window=0, q_pos=None, split_rows=0, scale=None):
    """q: float32 numpy [n_seq, hq, d]; segs_np: per seq list of (k_rows, v_rows, pos0)."""
    import torch
    from decode_attention_offloaded_amd import kvd
    qd = to_dev(q)
    out = torch.full_like(qd, float("nan"))
    segs = [[(to_dev(k), to_dev(v), p0) for (k, v, p0) in seq] for seq in segs_np]
    kvd.attend_decode(qd, out, segs, n_head_kv, window=window, q_pos=q_pos, split_rows=split_rows, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()
