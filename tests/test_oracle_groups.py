"""Pins of the oracle's group composition (the DiTango page, State-Centric
Parallel Runtime > Dynamic Group Compose): composed group states checked against
attention over the members' concatenated K/V, recursive composition against
direct composition, and the step's whole-group reuse rule against steps run
without groups."""

import numpy as np
import pytest

from oracle import (StateCache, attn_step, compose_runs, effective_reuse, full_attention, merge_states,
                    partial_state)


def _parts(rng, nq, d, lengths, scale=1.5):
    q = rng.standard_normal((2, nq, d)) * scale
    ks = [rng.standard_normal((2, n, d)) * scale for n in lengths]
    vs = [rng.standard_normal((2, n, d)) for n in lengths]
    return q, ks, vs


def _filled(q, ks, vs, step=0):
    cache = StateCache(len(ks))
    o, lse, nf = attn_step(cache, q, ks, vs, np.zeros(len(ks), np.uint8), step)
    assert nf == len(ks)
    return cache, o, lse


def test_group_state_is_attention_over_members():
    rng = np.random.default_rng(0)
    q, ks, vs = _parts(rng, 7, 8, [5, 3, 9, 4, 6])
    cache, _, _ = _filled(q, ks, vs)
    cache.compose(1, 3)
    o_ref, lse_ref = full_attention(q, ks[1:4], vs[1:4])
    o, lse = cache.slots[1]
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
    assert cache.slots[2] is None and cache.slots[3] is None
    assert list(cache.group) == [0, 1, 1, 1, 4]
    assert cache.group_range(2) == (1, 3) and cache.live_states() == 3


def test_recursive_compose_equals_direct_compose():
    rng = np.random.default_rng(1)
    q, ks, vs = _parts(rng, 6, 4, [4, 4, 4, 4, 4, 4, 4, 4])
    a, _, _ = _filled(q, ks, vs)
    b, _, _ = _filled(q, ks, vs)
    for i in range(0, 8, 2):
        a.compose(i, i + 1)
    a.compose(0, 3)
    a.compose(4, 7)
    a.compose(0, 7)
    b.compose(0, 7)
    o_ref, lse_ref = full_attention(q, ks, vs)
    for c in (a, b):
        o, lse = c.slots[0]
        assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
        assert c.live_states() == 1


def test_all_reuse_step_unchanged_by_composition():
    rng = np.random.default_rng(2)
    q, ks, vs = _parts(rng, 9, 8, [6, 6, 6, 6, 6])
    cache, o0, lse0 = _filled(q, ks, vs)
    cache.compose(2, 4)
    o, lse, nf = attn_step(cache, q, ks, vs, np.ones(5, np.uint8), 1)
    assert nf == 0
    assert np.max(np.abs(o - o0)) < 1e-12 and np.max(np.abs(lse - lse0)) < 1e-12


def test_partial_reuse_recomputes_and_dissolves_the_group():
    rng = np.random.default_rng(3)
    q, ks, vs = _parts(rng, 5, 4, [3, 5, 4, 6])
    cache, _, _ = _filled(q, ks, vs, step=0)
    cache.compose(1, 3)
    old0 = cache.slots[0]
    # new K/V for step 1; partition 2 alone is marked fresh, so 1..3 are all recomputed
    q2, ks2, vs2 = _parts(np.random.default_rng(4), 5, 4, [3, 5, 4, 6])
    mask = np.array([1, 1, 0, 1], np.uint8)
    assert list(effective_reuse(cache, mask)) == [1, 0, 0, 0]
    o, lse, nf = attn_step(cache, q, ks2, vs2, mask, 1)
    assert nf == 3 and list(cache.group) == [0, 1, 2, 3] and list(cache.stamp) == [0, 1, 1, 1]
    ref = merge_states([old0] + [partial_state(q, ks2[p], vs2[p]) for p in (1, 2, 3)])
    assert np.max(np.abs(o - ref[0])) < 1e-12 and np.max(np.abs(lse - ref[1])) < 1e-12


def test_group_stamp_is_the_oldest_member():
    rng = np.random.default_rng(5)
    q, ks, vs = _parts(rng, 4, 4, [3, 3, 3])
    cache = StateCache(3)
    attn_step(cache, q, ks, vs, np.zeros(3, np.uint8), 4)
    attn_step(cache, q, ks, vs, np.array([1, 0, 1], np.uint8), 7)
    cache.compose(0, 2)
    assert list(cache.stamp) == [4, 4, 4]


def test_compose_rejects_bad_ranges():
    rng = np.random.default_rng(6)
    q, ks, vs = _parts(rng, 3, 4, [2, 2, 2, 2])
    cache, _, _ = _filled(q, ks, vs)
    with pytest.raises(ValueError):
        cache.compose(2, 1)
    with pytest.raises(ValueError):
        cache.compose(0, 4)
    cache.compose(1, 2)
    with pytest.raises(ValueError):
        cache.compose(2, 3)          # straddles the group [1, 2]
    with pytest.raises(RuntimeError):
        cache.store(2, cache.slots[1], 3)
    cache.invalidate(2)              # dissolves and empties the whole group
    assert list(cache.valid) == [1, 0, 0, 1] and list(cache.group) == [0, 1, 2, 3]
    with pytest.raises(RuntimeError):
        cache.compose(0, 1)          # partition 1 holds no state


def test_compose_runs_then_step_reuses_exactly_the_mask():
    """Composing the next mask's reuse runs ahead of the step: the step then
    recomputes exactly the partitions the mask marks fresh, reads one state per
    run, and its output is the merge of new fresh states and old reused ones."""
    rng = np.random.default_rng(7)
    lengths = [4, 6, 3, 5, 7, 2, 4, 6]
    q, ks0, vs0 = _parts(rng, 5, 4, lengths)
    _, ks1, vs1 = _parts(np.random.default_rng(8), 5, 4, lengths)
    cache, _, _ = _filled(q, ks0, vs0, step=0)
    mask = np.array([0, 1, 1, 1, 0, 1, 0, 1], np.uint8)   # runs [1,3], [5,5], [7,7]
    assert compose_runs(cache, mask) == 1
    assert [cache.group_range(p) for p in range(8)] == [
        (0, 0), (1, 3), (1, 3), (1, 3), (4, 4), (5, 5), (6, 6), (7, 7)]
    o, lse, nf = attn_step(cache, q, ks1, vs1, mask, 1)
    assert nf == 3 and cache.live_states() == 6
    states = [partial_state(q, ks1[p], vs1[p]) if mask[p] == 0 else partial_state(q, ks0[p], vs0[p])
              for p in range(8)]
    ref = merge_states(states)
    assert np.max(np.abs(o - ref[0])) < 1e-12 and np.max(np.abs(lse - ref[1])) < 1e-12
    # the run is already one group: nothing more to compose
    assert compose_runs(cache, mask) == 0


def test_compose_runs_leaves_out_groups_reaching_outside():
    rng = np.random.default_rng(9)
    q, ks, vs = _parts(rng, 3, 4, [3] * 7)
    cache, _, _ = _filled(q, ks, vs)
    cache.compose(1, 3)
    cache.compose(5, 6)
    # run [2,5]: group [1,3] reaches left of it and [5,6] right of it -> only [4,4] left: no-op
    assert compose_runs(cache, np.array([0, 0, 1, 1, 1, 1, 0], np.uint8)) == 0
    assert cache.group_range(4) == (4, 4)
    # run [1,6] holds both groups and partition 4: one composition of three states
    assert compose_runs(cache, np.array([0, 1, 1, 1, 1, 1, 1], np.uint8)) == 1
    assert cache.group_range(2) == (1, 6) and cache.live_states() == 2
    with pytest.raises(RuntimeError):
        cache.invalidate(0)
        compose_runs(cache, np.array([1, 0, 0, 0, 0, 0, 0], np.uint8))


def test_any_schedule_of_groups_on_fixed_inputs_is_full_attention():
    """With K/V unchanged between steps, every state -- fresh, reused or composed
    -- is a piece of the same attention, so any sequence of masks, compositions
    and recomputations must return full attention."""
    rng = np.random.default_rng(10)
    q, ks, vs = _parts(rng, 6, 4, [3, 5, 2, 6, 4, 3, 5, 2, 4])
    o_ref, lse_ref = full_attention(q, ks, vs)
    cache = StateCache(9)
    attn_step(cache, q, ks, vs, np.zeros(9, np.uint8), 0)
    for s in range(1, 25):
        mask = (rng.random(9) < 0.7).astype(np.uint8)
        compose_runs(cache, mask)
        o, lse, nf = attn_step(cache, q, ks, vs, mask, s)
        assert nf >= int((mask == 0).sum())      # groups straddling a fresh run are recomputed
        assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
        if s % 4 == 0:
            a = int(rng.integers(0, 8))
            b = int(rng.integers(a, 9))
            try:
                cache.compose(a, b)
            except ValueError:
                pass        # a group straddles [a, b]
