"""Residency planner (host-only): which layers stay on the device, whether
the rest go through a ring.  Pinned by the scenarios the pages describe and
by a brute-force search over every (resident count, ring or not) candidate."""
import itertools

import pytest

from decode_attention_offloaded_amd import kvd

LAYER = 2 * 131072 * 1088     # K+V of one 131072-row layer, 8 KV heads x 128, q8_0
MiB, GiB = 1 << 20, 1 << 30


def _est(n_layers, k, lb, ring, bw, c):
    """Step-time estimate as the header states it (transfer-bound model)."""
    t_x = (n_layers - k) * lb / (bw * 1e6)
    t_c = n_layers * c
    if not ring or k == n_layers:
        return t_x + t_c
    return max(t_x, t_c) + max(0.0, lb / (bw * 1e6) - k * c)


def test_everything_resident_when_it_fits():
    p = kvd.plan_residency(16, LAYER, 16 * LAYER, 1, 57.0, 0.2)
    assert p["n_resident"] == 16 and p["use_ring"] == 0 and p["staged_bytes_per_step"] == 0
    assert p["ring_bytes"] == 0 and p["resident_bytes"] == 16 * LAYER


def test_pages_scenario_three_resident_layers_beat_the_ring():
    """16 attention layers at 131072 rows, a budget the size of a depth-1 ring
    (3 layers): resident layers remove 3/16 of the transfer (~19%) while the
    ring hides only the compute, which is small here."""
    budget = 3 * LAYER
    p = kvd.plan_residency(16, LAYER, budget, 1, 57.0, 0.2)
    assert p["n_resident"] == 3 and p["use_ring"] == 0
    assert p["staged_bytes_per_step"] == 13 * LAYER
    # with compute as long as the transfer, overlap wins instead
    q = kvd.plan_residency(16, LAYER, budget, 1, 57.0, LAYER / 57e6)
    assert q["use_ring"] == 1 and q["n_resident"] == 0


def test_without_a_model_the_ring_is_kept_when_it_fits():
    p = kvd.plan_residency(64, LAYER, 1 * GiB, 1, 0.0, 0.0)
    assert p["use_ring"] == 1 and p["n_resident"] == 0 and p["ring_bytes"] == 3 * LAYER
    p = kvd.plan_residency(64, LAYER, 4 * GiB, 1, 0.0, 0.0)
    assert p["use_ring"] == 1 and p["n_resident"] == (4 * GiB - 3 * LAYER) // LAYER
    # the ring does not fit: ordered, with what fits resident
    p = kvd.plan_residency(64, LAYER, 128 * MiB, 1, 0.0, 0.0)
    assert p["use_ring"] == 0 and p["n_resident"] == 0 and p["staged_bytes_per_step"] == 64 * LAYER
    p = kvd.plan_residency(64, LAYER, 700 * MiB, 1, 0.0, 0.0)
    assert p["use_ring"] == 0 and p["n_resident"] == 2


@pytest.mark.parametrize("n_layers,depth", [(1, 1), (7, 1), (16, 2), (64, 1), (64, 0)])
def test_model_choice_is_the_best_candidate(n_layers, depth):
    lb = 35_651_584   # one 16384-row layer
    for budget_layers, bw, c in itertools.product((0, 1, 2.5, 3, 5, 20, 70), (25.0, 57.0), (0.01, 0.1, 0.7, 2.0)):
        budget = int(budget_layers * lb)
        p = kvd.plan_residency(n_layers, lb, budget, depth, bw, c)
        if n_layers * lb <= budget:
            assert p["n_resident"] == n_layers and p["use_ring"] == 0
            continue
        cands = []
        ring = (depth + 2) * lb if depth else None
        if ring is not None and budget >= ring:
            k = min(n_layers, (budget - ring) // lb)
            if k < n_layers:
                cands.append((_est(n_layers, k, lb, True, bw, c), k, 1))
        k = min(n_layers, budget // lb)
        cands.append((_est(n_layers, k, lb, False, bw, c), k, 0))
        t_best = min(t for t, _, _ in cands)
        got = _est(n_layers, p["n_resident"], lb, bool(p["use_ring"]), bw, c)
        assert abs(got - t_best) <= 1e-9 * max(1.0, t_best), (budget_layers, bw, c, p, cands)
        assert abs(p["est_ms_per_step"] - got) <= 1e-9 * max(1.0, got)
        assert p["resident_bytes"] + p["ring_bytes"] <= budget


@pytest.mark.parametrize("args", [(0, LAYER, GiB, 1, 0.0, 0.0), (4, 0, GiB, 1, 0.0, 0.0), (4, LAYER, GiB, -1, 0.0, 0.0),
                                  (4, LAYER, GiB, 1, -1.0, 0.0), (4, LAYER, GiB, 1, 1.0, float("nan")),
                                  (4, LAYER, GiB, 1, float("inf"), 0.0)])
def test_bad_arguments(args):
    with pytest.raises(kvd.KvdError):
        kvd.plan_residency(*args)
