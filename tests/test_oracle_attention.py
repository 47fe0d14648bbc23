"""Pins of the oracle's partial attention state (CPU only).

Each test ties ``oracle.partial_state`` to something other than itself:
an independent library routine, a closed form, or brute-force scalar loops.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import full_attention, partial_state, softmax_scale


def _rand(rng, *shape, scale=1.0):
    return scale * rng.standard_normal(shape)


@pytest.mark.parametrize("nq,nk,d", [(1, 1, 1), (3, 7, 4), (17, 33, 16), (64, 300, 64), (5, 129, 128)])
def test_lse_matches_scipy_logsumexp(nq, nk, d):
    rng = np.random.default_rng(nq * 1000 + nk)
    q, k, v = _rand(rng, 2, nq, d, scale=2.0), _rand(rng, 2, nk, d, scale=2.0), _rand(rng, 2, nk, d)
    tau = softmax_scale(d)
    _, lse = partial_state(q, k, v)
    s = tau * np.einsum("hid,hjd->hij", q, k)
    ref = scipy.special.logsumexp(s, axis=-1)
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("nq,nk,d", [(4, 9, 8), (33, 65, 64), (16, 257, 128)])
def test_output_matches_torch_sdpa_fp64(nq, nk, d):
    rng = np.random.default_rng(7 + nk)
    q, k, v = _rand(rng, 1, 3, nq, d), _rand(rng, 1, 3, nk, d), _rand(rng, 1, 3, nk, d)
    o, _ = partial_state(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_explicit_scale_is_used():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 5, 8), _rand(rng, 11, 8), _rand(rng, 11, 8)
    o1, l1 = partial_state(q, k, v, scale=0.7)
    o2, l2 = partial_state(0.7 * q, k, v, scale=1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_zero_queries_closed_form():
    # Q = 0: every score is 0, so LSE = ln Nk and O = mean of the value rows.
    rng = np.random.default_rng(11)
    nk, d = 37, 16
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    o, lse = partial_state(np.zeros((6, d)), k, v)
    np.testing.assert_allclose(lse, np.full(6, math.log(nk)), atol=1e-14)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (6, 1)), atol=1e-14)


def test_identical_keys_closed_form():
    # All key rows equal k: LSE_i = tau q_i.k + ln Nk, O = mean of the value rows.
    rng = np.random.default_rng(12)
    nq, nk, d = 9, 23, 32
    q, kr, v = _rand(rng, nq, d), _rand(rng, d), _rand(rng, nk, d)
    k = np.tile(kr, (nk, 1))
    o, lse = partial_state(q, k, v)
    tau = 1.0 / math.sqrt(d)
    np.testing.assert_allclose(lse, tau * q @ kr + math.log(nk), atol=1e-12)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (nq, 1)), atol=1e-13)


def test_constant_values_closed_form():
    # V rows all equal c: the softmax weights sum to 1, so O = c whatever the scores.
    rng = np.random.default_rng(13)
    c = _rand(rng, 8)
    q, k = _rand(rng, 7, 8, scale=3.0), _rand(rng, 40, 8, scale=3.0)
    o, _ = partial_state(q, k, np.tile(c, (40, 1)))
    np.testing.assert_allclose(o, np.tile(c, (7, 1)), atol=1e-13)


def test_single_key_closed_form():
    # Nk = 1: the state is (v, tau q.k).
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 5, 4), _rand(rng, 1, 4), _rand(rng, 1, 4)
    o, lse = partial_state(q, k, v)
    np.testing.assert_allclose(o, np.tile(v[0], (5, 1)), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * q @ k[0], atol=1e-15)


def test_output_rows_are_convex_combinations():
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 50, 16, scale=4.0), _rand(rng, 60, 16, scale=4.0), _rand(rng, 60, 16)
    o, _ = partial_state(q, k, v)
    assert np.all(o <= v.max(axis=0) + 1e-12) and np.all(o >= v.min(axis=0) - 1e-12)


def test_empty_partition_is_neutral():
    o, lse = partial_state(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 4)))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _brute_state(q, k, v, tau):
    """Scalar loops with exactly summed exponentials: the definition, element by element."""
    nq, d = q.shape
    nk = k.shape[0]
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        s = [tau * math.fsum(q[i, t] * k[j, t] for t in range(d)) for j in range(nk)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        lse[i] = m + math.log(den)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(e[j] * v[j, c] for j in range(nk)) / den
    return o, lse


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    nq, nk, d = rng.integers(1, 9), rng.integers(1, 9), rng.integers(1, 5)
    q, k, v = _rand(rng, nq, d, scale=3), _rand(rng, nk, d, scale=3), _rand(rng, nk, d)
    tau = softmax_scale(d)
    o, lse = partial_state(q, k, v)
    ob, lb = _brute_state(q, k, v, tau)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


def test_full_attention_is_attention_over_concatenation():
    rng = np.random.default_rng(16)
    q = _rand(rng, 4, 8)
    ks = [_rand(rng, n, 8) for n in (3, 5, 1)]
    vs = [_rand(rng, n, 8) for n in (3, 5, 1)]
    o, lse = full_attention(q, ks, vs)
    ob, lb = _brute_state(q, np.concatenate(ks), np.concatenate(vs), softmax_scale(8))
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)
