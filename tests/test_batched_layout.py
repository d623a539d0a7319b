"""Row bookkeeping of the batched mixed-residency stack, pinned by brute force."""
import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from decode_attention_offloaded_amd.batched import BatchedLayout, cfg4_lengths

RB = 1088


def _visible(n, window):
    """Positions visible from the query at n - 1 (brute force)."""
    q = n - 1
    return {p for p in range(n) if p <= q and (window == 0 or q - p < window)}


@pytest.mark.parametrize("window", [0, 1, 7, 64, 300])
def test_staged_rows_are_exactly_the_visible_host_rows(window):
    rng = np.random.default_rng(5)
    lengths = rng.integers(2, 400, size=9)
    lay = BatchedLayout(lengths, n_layers=4, window=window, row_bytes=RB)
    for l in range(4):
        w = window if l % 2 == 1 else 0
        assert lay.window[l] == w
        off = 0
        for s, n in enumerate(lengths):
            h = n // 2
            staged = set(range(int(lay.lo[l][s]), int(lay.lo[l][s] + lay.stage_rows[l][s])))
            assert staged == {p for p in _visible(n, w) if p < h}
            # packed sequence-major, no gaps
            assert lay.stage_off[l][s] == off
            off += lay.stage_rows[l][s]
            # device half: every row from h on, newest row included
            assert lay.dev_rows[s] == n - h and lay.h[s] == h and lay.q_pos[s] == n - 1
        assert lay.stage_total[l] == off
    assert lay.cap_rows == max(max(lay.stage_total), 1)
    assert lay.host_layer_off[0] == 0
    assert all(lay.host_layer_off[l + 1] - lay.host_layer_off[l] == lay.stage_total[l] * RB for l in range(3))
    assert lay.host_bytes == sum(lay.stage_total) * RB


def test_byte_counts_match_brute_force():
    lengths = [2, 3, 100, 257, 1000]
    lay = BatchedLayout(lengths, n_layers=3, window=50, row_bytes=RB)
    staged = sum(len({p for p in _visible(n, lay.window[l]) if p < n // 2}) for l in range(3) for n in lengths)
    assert lay.staged_bytes_per_token() == 2 * staged * RB
    vis = sum(len(_visible(n, lay.window[l])) for l in range(3) for n in lengths)
    assert lay.visible_bytes_per_token() == 2 * vis * RB


def test_window_past_the_host_half_stages_nothing():
    # n >= 2W: the window starts inside the device half
    lay = BatchedLayout([4096, 8192, 9000], n_layers=2, window=4096, row_bytes=RB)
    assert list(lay.stage_rows[1]) == [2048, 0, 0]
    assert list(lay.stage_rows[0]) == [2048, 4096, 4500]


def test_too_short_sequences_are_rejected():
    with pytest.raises(ValueError):
        BatchedLayout([1, 5], n_layers=1, window=0, row_bytes=RB)


def test_batched_lengths_follow_the_recipe():
    cfg = inputs.config(4)
    a, b = cfg4_lengths(cfg), cfg4_lengths(cfg)
    assert len(a) == 16 and (a == b).all()
    assert a.min() >= 1024 and a.max() <= 32768
    # lognormal around 4096: the sample median sits within a factor 2 of it
    assert 2048 <= np.median(a) <= 8192
