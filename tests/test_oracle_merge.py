"""Pins of the oracle's LSE merge and rank-step (CPU only).

The DiTango page (Methodology > State-Centric Parallel Runtime > State
Composition) says attention states compose associatively and commutatively;
the softmax algebra adds that merging all-fresh partition states gives full
attention over the concatenated sequence.  These tests pin the oracle to
those facts and to closed forms.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import StateCache, attn_step, full_attention, merge_states, partial_state


def _parts(rng, nq, d, lengths, scale=2.0):
    q = scale * rng.standard_normal((2, nq, d))
    ks = [scale * rng.standard_normal((2, n, d)) for n in lengths]
    vs = [rng.standard_normal((2, n, d)) for n in lengths]
    return q, ks, vs


@pytest.mark.parametrize("lengths", [(8,), (5, 9), (16, 16, 16, 16), (1, 30, 7, 2, 11), (64,) * 8])
def test_all_fresh_merge_equals_full_attention(lengths):
    rng = np.random.default_rng(len(lengths) * 31 + sum(lengths))
    q, ks, vs = _parts(rng, 13, 16, lengths)
    states = [partial_state(q, k, v) for k, v in zip(ks, vs)]
    o, lse = merge_states(states)
    of, lf = full_attention(q, ks, vs)
    np.testing.assert_allclose(o, of, atol=1e-12)
    np.testing.assert_allclose(lse, lf, atol=1e-12)


def test_merge_is_associative_and_order_independent():
    rng = np.random.default_rng(5)
    q, ks, vs = _parts(rng, 9, 8, (4, 6, 3, 5))
    st = [partial_state(q, k, v) for k, v in zip(ks, vs)]
    ref_o, ref_l = merge_states(st)
    left = merge_states([merge_states([merge_states(st[:2]), st[2]]), st[3]])
    right = merge_states([st[0], merge_states([st[1], merge_states(st[2:])])])
    pairs = merge_states([merge_states(st[:2]), merge_states(st[2:])])
    for o, l in (left, right, pairs):
        np.testing.assert_allclose(o, ref_o, atol=1e-12)
        np.testing.assert_allclose(l, ref_l, atol=1e-12)
    for perm in itertools.permutations(range(4)):
        o, l = merge_states([st[i] for i in perm])
        np.testing.assert_allclose(o, ref_o, atol=1e-12)
        np.testing.assert_allclose(l, ref_l, atol=1e-12)


def test_single_state_is_identity():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((3, 5, 8))
    lse = 4 * rng.standard_normal((3, 5))
    mo, ml = merge_states([(o, lse)])
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, lse, atol=1e-15)


def test_neutral_state_changes_nothing():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((5, 8))
    lse = rng.standard_normal(5)
    neutral = (rng.standard_normal((5, 8)), np.full(5, -np.inf))
    mo, ml = merge_states([neutral, (o, lse), neutral])
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, lse, atol=1e-15)


def test_all_neutral_rows_merge_to_zero_and_minus_inf():
    o = np.ones((2, 4))
    lse = np.array([-np.inf, 1.0])
    mo, ml = merge_states([(o, lse), (2 * o, np.array([-np.inf, 1.0]))])
    assert np.all(mo[0] == 0) and np.isneginf(ml[0])
    np.testing.assert_allclose(mo[1], 1.5 * np.ones(4), atol=1e-15)
    np.testing.assert_allclose(ml[1], 1.0 + math.log(2.0), atol=1e-15)


def test_equal_lse_closed_form():
    # Two states with equal LSE: O is their average, LSE grows by ln 2.
    rng = np.random.default_rng(8)
    a, b = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    lse = 3 * rng.standard_normal(6)
    mo, ml = merge_states([(a, lse), (b, lse.copy())])
    np.testing.assert_allclose(mo, 0.5 * (a + b), atol=1e-14)
    np.testing.assert_allclose(ml, lse + math.log(2.0), atol=1e-14)


def test_weights_follow_lse_gap_closed_form():
    # LSE_b = LSE_a + ln 3: weights 1/4 and 3/4; LSE = LSE_a + ln 4.
    rng = np.random.default_rng(9)
    a, b = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    la = rng.standard_normal(4)
    mo, ml = merge_states([(a, la), (b, la + math.log(3.0))])
    np.testing.assert_allclose(mo, 0.25 * a + 0.75 * b, atol=1e-14)
    np.testing.assert_allclose(ml, la + math.log(4.0), atol=1e-14)


def test_group_compose_then_merge():
    # Cached states merged into coarser groups merge to the same result.
    rng = np.random.default_rng(10)
    q, ks, vs = _parts(rng, 7, 8, (3,) * 6)
    st = [partial_state(q, k, v) for k, v in zip(ks, vs)]
    groups = [merge_states(st[0:2]), merge_states(st[2:5]), st[5]]
    o, l = merge_states(groups)
    of, lf = full_attention(q, ks, vs)
    np.testing.assert_allclose(o, of, atol=1e-12)
    np.testing.assert_allclose(l, lf, atol=1e-12)


# ---------------------------------------------------------------- rank-step


def test_step_all_fresh_equals_full_attention_and_all_reuse_reproduces():
    rng = np.random.default_rng(20)
    q, ks, vs = _parts(rng, 6, 8, (5,) * 4)
    cache = StateCache(4)
    o0, l0, nf = attn_step(cache, q, ks, vs, [0, 0, 0, 0], step=0)
    assert nf == 4 and list(cache.stamp) == [0] * 4
    of, lf = full_attention(q, ks, vs)
    np.testing.assert_allclose(o0, of, atol=1e-12)
    np.testing.assert_allclose(l0, lf, atol=1e-12)
    # New K/V, but every partition reused: the output is exactly the cached one.
    ks2 = [k + 1.0 for k in ks]
    o1, l1, nf = attn_step(cache, q, ks2, vs, [1, 1, 1, 1], step=1)
    assert nf == 0 and list(cache.stamp) == [0] * 4
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)


def test_step_mixed_mask_uses_old_states_for_reused_partitions():
    rng = np.random.default_rng(21)
    q, ks, vs = _parts(rng, 6, 8, (4, 6, 5))
    cache = StateCache(3)
    attn_step(cache, q, ks, vs, [0, 0, 0], step=0)
    ks2 = [k + 0.3 * rng.standard_normal(k.shape) for k in ks]
    vs2 = [v + 0.3 * rng.standard_normal(v.shape) for v in vs]
    o, l, nf = attn_step(cache, q, ks2, vs2, [0, 1, 0], step=1)
    assert nf == 2 and list(cache.stamp) == [1, 0, 1]
    expect = merge_states([partial_state(q, ks2[0], vs2[0]), partial_state(q, ks[1], vs[1]),
                           partial_state(q, ks2[2], vs2[2])])
    np.testing.assert_allclose(o, expect[0], atol=1e-12)
    np.testing.assert_allclose(l, expect[1], atol=1e-12)


def test_step_rejects_reuse_of_empty_slot():
    rng = np.random.default_rng(22)
    q, ks, vs = _parts(rng, 2, 4, (3, 3))
    with pytest.raises(RuntimeError):
        attn_step(StateCache(2), q, ks, vs, [0, 1], step=0)
