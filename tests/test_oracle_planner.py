"""Pins of the oracle's reuse-mask planner and its SplitMix64 generator (CPU only)."""

import os

import numpy as np
import pytest

import workloads
from oracle import (POLICY_DIST, POLICY_KNEAREST, POLICY_RAMP, POLICY_RANDOM, Plan,
                    SplitMix64, plan_mask, radius_at)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_splitmix64_published_first_output():
    for seed, hexval, signed in _golden_rows("splitmix64_seed0.txt"):
        g = SplitMix64(int(seed))
        x = g.next()
        assert x == int(hexval, 16)
        assert x - (1 << 64) == int(signed)


def test_splitmix64_state_advances_by_gamma():
    # Seeding at state s + gamma must give the second output of the stream seeded at s.
    g = SplitMix64(12345)
    g.next()
    second = g.next()
    assert SplitMix64(12345 + SplitMix64.GAMMA).next() == second


def _plan(name):
    wl = workloads.get(name)
    return wl, Plan(**wl.plan_fields())


def _run_schedule(name):
    """Masks of a workload's whole schedule with the cache filled as it goes."""
    wl, plan = _plan(name)
    valid = np.zeros(wl.P, np.uint8)
    masks = []
    for s in range(wl.steps):
        m = plan_mask(plan, s, valid)
        masks.append(m)
        valid[m == 0] = 1
    return masks


def _fresh(mask):
    return [p for p in range(len(mask)) if mask[p] == 0]


def test_tiny_schedule_fresh_partitions():
    # Queries = partition 0; recompute partitions at distance <= 1: {0, 1}.
    masks = _run_schedule("tiny_f32")
    assert _fresh(masks[0]) == [0, 1, 2, 3]          # cold cache
    assert _fresh(masks[1]) == [0, 1]


def test_dit32k_two_nearest_including_local():
    masks = _run_schedule("dit32k_bf16")
    assert _fresh(masks[1]) == [0, 1]


def test_dit75k_anchor_schedule_counts():
    masks = _run_schedule("dit75k_bf16")
    counts = [len(_fresh(m)) for m in masks]
    assert counts == [16, 3, 3, 3, 3, 16, 3, 3, 3, 3]
    assert sum(counts) == 56
    assert _fresh(masks[1]) == [0, 1, 2]


def test_ramp50_radius_schedule_and_fresh_total():
    wl, plan = _plan("dit75k_ramp50")
    radii = [radius_at(plan, s) for s in range(50)]
    # round(8 - 7 s / 49) for s = 0..49: 8 x4, 7..2 x7 each, 1 x4.
    expect = [8] * 4 + [7] * 7 + [6] * 7 + [5] * 7 + [4] * 7 + [3] * 7 + [2] * 7 + [1] * 4
    assert radii == expect
    for s in range(50):
        assert radii[s] == int(np.floor(8 - 7 * s / 49 + 0.5))
    masks = _run_schedule("dit75k_ramp50")
    counts = [len(_fresh(m)) for m in masks]
    assert counts[0] == 16
    assert counts[1:] == [min(r, 15) + 1 for r in radii[1:]]
    assert sum(counts) == 282


def test_local_partition_always_fresh_and_anchor_all_fresh():
    rng = np.random.default_rng(0)
    for _ in range(300):
        P = int(rng.integers(1, 65))
        plan = Plan(P=P, q=int(rng.integers(0, P)), policy=int(rng.integers(0, 4)),
                    radius=int(rng.integers(0, 6)), radius_end=int(rng.integers(0, 6)),
                    k_nearest=int(rng.integers(0, P + 1)), anchor_period=int(rng.integers(0, 4)),
                    total_steps=int(rng.integers(1, 30)), seed=int(rng.integers(0, 2**63)))
        s = int(rng.integers(0, 40))
        m = plan_mask(plan, s)
        assert m[plan.q] == 0
        if plan.anchor_period and s % plan.anchor_period == 0:
            assert not m.any()


def test_cold_slots_are_fresh():
    plan = Plan(P=6, q=2, policy=POLICY_DIST, radius=0)
    m = plan_mask(plan, 3, valid=[1, 0, 1, 1, 0, 1])
    assert list(m) == [1, 0, 0, 1, 0, 1]


def test_knearest_ties_go_to_lower_index():
    plan = Plan(P=8, q=3, policy=POLICY_KNEAREST, k_nearest=2)
    assert _fresh(plan_mask(plan, 1)) == [2, 3]
    plan = Plan(P=8, q=3, policy=POLICY_KNEAREST, k_nearest=3)
    assert _fresh(plan_mask(plan, 1)) == [2, 3, 4]


def test_random_policy_is_fair_and_deterministic():
    plan = Plan(P=64, q=0, policy=POLICY_RANDOM, seed=1)
    masks = np.stack([plan_mask(plan, s) for s in range(400)])
    frac = masks[:, 1:].mean()
    assert abs(frac - 0.5) < 0.02
    assert np.array_equal(masks[17], plan_mask(plan, 17))
    # Each step's stream is seeded with (seed << 32) ^ step; draw p is reuse iff its top bit is set.
    g = SplitMix64((1 << 32) ^ 17)
    assert list(masks[17][1:]) == [g.next() >> 63 for _ in range(64)][1:]


def test_distance_policy_radius():
    plan = Plan(P=9, q=4, policy=POLICY_DIST, radius=2)
    assert _fresh(plan_mask(plan, 1)) == [2, 3, 4, 5, 6]


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        plan_mask(Plan(P=0, q=0), 0)
    with pytest.raises(ValueError):
        plan_mask(Plan(P=65, q=0), 0)
    with pytest.raises(ValueError):
        plan_mask(Plan(P=4, q=4), 0)
    with pytest.raises(ValueError):
        plan_mask(Plan(P=4, q=0, policy=9), 0)
