"""Pins of the oracle's error-guided planner (the DiTango page, Methodology >
1. Anchor-Guided Selection Planner): contribution weights against the softmax
algebra, the local-change measure against closed forms, and the group choice
against a hand-worked case and brute force over subsets."""

import itertools
import math

import numpy as np
import pytest

from oracle import full_attention, merge_states, partial_state
from oracle.error_planner import ErrorPlanner, contributions, state_change


def test_contributions_sum_to_one_and_match_the_softmax_mass():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 9, 8))
    ks = [rng.standard_normal((2, n, 8)) for n in (5, 3, 7, 4)]
    vs = [rng.standard_normal((2, n, 8)) for n in (5, 3, 7, 4)]
    states = [partial_state(q, k, v) for k, v in zip(ks, vs)]
    _, lse = merge_states(states)
    w = contributions([l for _, l in states], lse)
    assert abs(w.sum() - 1.0) < 1e-12
    # brute force: the share of each partition in the full softmax, row by row
    s = np.concatenate([q @ k.swapaxes(-1, -2) for k in ks], axis=-1) / math.sqrt(8)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    edges = np.cumsum([0, 5, 3, 7, 4])
    share = [p[..., a:b].sum(-1).mean() for a, b in zip(edges[:-1], edges[1:])]
    assert np.max(np.abs(w - np.array(share))) < 1e-12


def test_contributions_closed_forms():
    # identical partitions share equally
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 4, 4))
    k = rng.standard_normal((1, 6, 4))
    v = rng.standard_normal((1, 6, 4))
    st = [partial_state(q, k, v)] * 5
    w = contributions([l for _, l in st], full_attention(q, [k] * 5, [v] * 5)[1])
    assert np.max(np.abs(w - 0.2)) < 1e-12
    # two states whose LSEs differ by ln 3 on every row: 3/4 and 1/4
    lse_a = np.array([0.3, -1.0, 2.0])
    lse_b = lse_a - math.log(3.0)
    lse = lse_a + math.log(4.0 / 3.0)
    w = contributions([lse_a, lse_b], lse)
    assert np.max(np.abs(w - [0.75, 0.25])) < 1e-12
    # an all -inf row counts zero for everyone
    w = contributions([np.array([0.0, -np.inf]), np.array([0.0, -np.inf])],
                      np.array([math.log(2.0), -np.inf]))
    assert np.max(np.abs(w - [0.25, 0.25])) < 1e-12


def test_state_change_closed_forms():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((3, 5, 4))
    assert state_change(a, a) == 0.0
    assert abs(state_change(1.25 * a, a) - 0.25) < 1e-12
    assert abs(state_change(-a, a) - 2.0) < 1e-12
    e1 = np.zeros((2, 2)); e1[0, 0] = 3.0
    e2 = np.zeros((2, 2)); e2[1, 1] = 3.0
    assert abs(state_change(e2, e1) - math.sqrt(2.0)) < 1e-15
    assert state_change(np.zeros(3), np.zeros(3)) == 0.0
    assert state_change(np.ones(3), np.zeros(3)) == math.inf


def _planner():
    pl = ErrorPlanner(P=6, q=0, group_size=2, budget=0.016, anchor_period=5)
    pl.set_weights([0.4, 0.2, 0.15, 0.15, 0.05, 0.05])
    pl.observe(1, 0.01)
    pl.observe(2, 0.02)
    return pl


def test_hand_worked_case():
    """Step 3, stamps [2,0,0,1,0,0]; delta 0.01 at step 1, 0.02 at step 2, and
    0.02 predicted for step 3.  Growth since stamp 0: 0.05; since stamp 1: 0.04.
    Errors [0, .01, .0075, .006, .0025, .0025]; groups {1}: .01, {2,3}: .0135,
    {4,5}: .005.  Budget .016 takes {4,5} then {1} (.015) and stops at {2,3}."""
    pl = _planner()
    valid = [1] * 6
    stamp = [2, 0, 0, 1, 0, 0]
    reuse, err = pl.mask(3, valid, stamp)
    assert np.max(np.abs(err - [0, 0.01, 0.0075, 0.006, 0.0025, 0.0025])) < 1e-15
    assert list(reuse) == [0, 1, 0, 0, 1, 1]
    # a looser budget takes every group; a zero budget none
    pl.budget = 0.03
    assert list(pl.mask(3, valid, stamp)[0]) == [0, 1, 1, 1, 1, 1]
    pl.budget = 0.0
    assert list(pl.mask(3, valid, stamp)[0]) == [0] * 6


def test_forced_fresh_cases():
    pl = _planner()
    valid, stamp = [1] * 6, [2, 0, 0, 1, 0, 0]
    assert list(pl.mask(5, valid, stamp)[0]) == [0] * 6          # anchor
    fresh = ErrorPlanner(P=6, q=0, group_size=2, budget=1.0)
    fresh.set_weights([1 / 6] * 6)
    assert list(fresh.mask(3, valid, stamp)[0]) == [0] * 6       # nothing observed yet
    unweighted = ErrorPlanner(P=6, q=0, group_size=2, budget=1.0)
    unweighted.observe(1, 0.1)
    assert list(unweighted.mask(3, valid, stamp)[0]) == [0] * 6  # no weights yet
    pl.budget = 1.0
    assert list(pl.mask(3, [1, 1, 1, 0, 1, 1], stamp)[0]) == [0, 1, 0, 0, 1, 1]  # cold member
    # the local partition is never reused, whatever its group does
    mid = ErrorPlanner(P=6, q=3, group_size=2, budget=1.0)
    mid.set_weights([0.1] * 6)
    mid.observe(0, 0.01)
    r, e = mid.mask(2, valid, [0] * 6)
    assert r[3] == 0 and e[3] == 0.0 and r[2] == 1


def test_prediction_uses_latest_observation():
    pl = ErrorPlanner(P=3, q=0, group_size=1, budget=10.0)
    pl.set_weights([0.0, 1.0, 1.0])
    pl.observe(4, 0.1)
    pl.observe(6, 0.3)
    # stamps 2 and 5 at step 8: t = 3..8 -> 0.1 (earliest, before any), 0.1, 0.1, 0.3, 0.3, 0.3
    _, err = pl.mask(8, [1, 1, 1], [0, 2, 5])
    assert abs(err[1] - (0.1 * 3 + 0.3 * 3)) < 1e-15
    assert abs(err[2] - 0.3 * 3) < 1e-15
    # an observation at the step itself is not yet known when planning it
    pl.observe(8, 5.0)
    _, err2 = pl.mask(8, [1, 1, 1], [0, 2, 5])
    assert np.array_equal(err, err2)


def test_choice_is_the_largest_cheapest_set_of_groups():
    """Brute force: the reused groups are a largest subset with total error within
    the budget, and among those one of least total error."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        P = int(rng.integers(2, 12))
        g = int(rng.integers(1, 4))
        q = int(rng.integers(0, P))
        pl = ErrorPlanner(P=P, q=q, group_size=g, budget=float(rng.uniform(0, 0.05)))
        pl.set_weights(list(rng.dirichlet(np.ones(P))))
        pl.observe(0, float(rng.uniform(0, 0.02)))
        valid = (rng.random(P) < 0.9).astype(np.uint8)
        stamp = rng.integers(0, 3, P)
        reuse, err = pl.mask(3, valid, stamp)
        groups = pl.groups()
        eligible = []
        for a, b in groups:
            mem = [p for p in range(a, b + 1) if p != q]
            if mem and all(valid[p] for p in mem):
                eligible.append((sum(err[p] for p in mem), mem))
        chosen = [mem for e, mem in eligible if all(reuse[p] for p in mem)]
        best_n, best_e = 0, 0.0
        for n in range(len(eligible), 0, -1):
            fits = [sum(e for e, _ in c) for c in itertools.combinations(eligible, n)
                    if sum(e for e, _ in c) <= pl.budget]
            if fits:
                best_n, best_e = n, min(fits)
                break
        assert len(chosen) == best_n, trial
        assert abs(sum(sum(err[p] for p in mem) for mem in chosen) - best_e) < 1e-12, trial
        assert reuse[q] == 0
        assert all(reuse[p] == 0 for p in range(P) if not valid[p])


def test_bad_parameters():
    for kw in [dict(P=0, q=0, group_size=1, budget=0.1), dict(P=4, q=4, group_size=1, budget=0.1),
               dict(P=4, q=0, group_size=0, budget=0.1), dict(P=4, q=0, group_size=1, budget=-1.0)]:
        with pytest.raises(ValueError):
            ErrorPlanner(**kw)

    pl = ErrorPlanner(P=3, q=0, group_size=1, budget=0.1)
    for bad in ([0.5, 0.5], [0.5, -0.1, 0.6], [0.5, math.nan, 0.5], [math.inf, 0.0, 0.0]):
        with pytest.raises(ValueError):
            pl.set_weights(bad)
    for step, d in ((-1, 0.1), (2, -0.1), (2, math.inf), (2, math.nan)):
        with pytest.raises(ValueError):
            pl.observe(step, d)


def test_high_contribution_groups_are_computed():
    """With fresh_weight set, a group holding a partition of at least that weight is
    never reused, whatever the budget; the hand-worked case with fresh_weight 0.2
    keeps group {1} (weight 0.2) fresh and reuses the others within the budget."""
    pl = _planner()
    pl.fresh_weight = 0.2
    pl.budget = 1.0
    valid, stamp = [1] * 6, [2, 0, 0, 1, 0, 0]
    assert list(pl.mask(3, valid, stamp)[0]) == [0, 0, 1, 1, 1, 1]
    pl.fresh_weight = 0.15          # {2,3} holds weights 0.15 too
    assert list(pl.mask(3, valid, stamp)[0]) == [0, 0, 0, 0, 1, 1]
    pl.fresh_weight = 0.5           # nobody but the local partition reaches it
    assert list(pl.mask(3, valid, stamp)[0]) == [0, 1, 1, 1, 1, 1]
    with pytest.raises(ValueError):
        ErrorPlanner(P=4, q=0, group_size=1, budget=0.1, fresh_weight=-0.1)
