"""CPU checks of the GPU tests' harness: the head-chunked oracle is the oracle,
and the covering row sample reaches every query block and tile."""

import numpy as np

from gpu_util import HeadChunkedOracle, covering_rows
from oracle import StateCache, attn_step, compose_runs


def test_head_chunked_oracle_equals_whole_oracle():
    rng = np.random.default_rng(5)
    B, H, nq, D, P = 1, 5, 37, 16, 5
    lengths = [11, 7, 20, 3, 9]
    q = rng.standard_normal((B, H, nq, D))
    whole, chunked = StateCache(P), HeadChunkedOracle(P, H, chunk=2, workers=3)
    masks = [np.zeros(P, np.uint8), np.array([0, 0, 1, 1, 1], np.uint8),
             np.array([0, 1, 1, 0, 1], np.uint8), np.array([0, 0, 1, 1, 1], np.uint8)]
    for s, m in enumerate(masks):
        ks = [rng.standard_normal((B, H, n, D)) for n in lengths]
        vs = [rng.standard_normal((B, H, n, D)) for n in lengths]
        o1, l1, n1 = attn_step(whole, q, ks, vs, m, s)
        o2, l2, n2 = chunked.step(q, ks, vs, m, s)
        assert n1 == n2
        assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
        assert np.array_equal(whole.valid, chunked.valid)
        for p in np.flatnonzero(m == 0):
            a, b = whole.slots[p], chunked.slot(int(p))
            assert np.max(np.abs(a[0] - b[0])) < 1e-12 and np.max(np.abs(a[1] - b[1])) < 1e-12
        if s + 1 < len(masks):
            assert compose_runs(whole, masks[s + 1]) == chunked.compose_runs(masks[s + 1])
            assert whole.leaders() == chunked.leaders()


def test_covering_rows_reach_every_block_and_tile():
    for nq in (4725, 4095, 2048, 33, 1):
        r = covering_rows(nq)
        assert r.min() >= 0 and r.max() == nq - 1 and len(set(r)) == len(r)
        assert set(r // 32) == set(range((nq + 31) // 32))
        for t0 in range(0, nq, 512):
            assert t0 in r and min(t0 + 512, nq) - 1 in r
        if nq >= 1024:
            assert len(set(r % 32)) == 32
