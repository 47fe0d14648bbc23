"""Helpers shared by the GPU parity tests (not a test module)."""

from __future__ import annotations

import sys

import numpy as np

# Acceptance tolerances (max-abs): fp32 1e-5 on O and LSE; bf16 1e-2 on O, 1e-3 on LSE.
TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str, dev):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)      # exact: the values are bf16-representable
    return t.to(dev)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        raise AssertionError(f"shape {a.shape} vs {b.shape}")
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def assert_state_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str = ""):
    to, tl = TOL[dtype]
    eo, el = max_abs(o_gpu, o_ref), max_abs(lse_gpu, lse_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    assert eo <= to, f"{what}: O max-abs {eo:.3e} > {to:.0e}"
    assert el <= tl, f"{what}: LSE max-abs {el:.3e} > {tl:.0e}"
    return eo, el


class HeadChunkedOracle:
    """The oracle's state cache and rank-step run separately on chunks of heads.

    Heads never interact in the method (every state, merge and composition is per
    (batch, head, row)), so the oracle over all heads is the concatenation of the
    oracle over each chunk.  The chunks run in a thread pool (numpy releases the
    interpreter lock in its matrix products and element-wise kernels) with the
    BLAS limited to one thread per chunk.  Arithmetic is entirely the oracle's.
    """

    def __init__(self, P: int, n_heads: int, chunk: int = 1, workers: int = 16):
        from oracle import StateCache
        self.P = P
        self.chunks = [slice(a, min(a + chunk, n_heads)) for a in range(0, n_heads, chunk)]
        self.caches = [StateCache(P) for _ in self.chunks]
        self.workers = max(1, min(workers, len(self.chunks), _cpu_share()))

    def _map(self, fn):
        from concurrent.futures import ThreadPoolExecutor
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        ctx = threadpool_limits(1) if threadpool_limits else _Null()
        with ctx, ThreadPoolExecutor(self.workers) as ex:
            return list(ex.map(fn, range(len(self.chunks))))

    @property
    def valid(self):
        return self.caches[0].valid

    def leaders(self):
        return self.caches[0].leaders()

    def group_range(self, p):
        return self.caches[0].group_range(p)

    def step(self, q, k_parts, v_parts, mask, s):
        from oracle import attn_step

        def one(i):
            sl = self.chunks[i]
            return attn_step(self.caches[i], q[:, sl], [x[:, sl] for x in k_parts],
                             [x[:, sl] for x in v_parts], mask, s)
        res = self._map(one)
        nf = {r[2] for r in res}
        assert len(nf) == 1
        return (np.concatenate([r[0] for r in res], axis=1),
                np.concatenate([r[1] for r in res], axis=1), nf.pop())

    def compose_runs(self, mask):
        from oracle import compose_runs
        res = self._map(lambda i: compose_runs(self.caches[i], mask))
        assert len(set(res)) == 1
        return res[0]

    def slot(self, p):
        st = [c.slots[p] for c in self.caches]
        return (np.concatenate([x[0] for x in st], axis=1),
                np.concatenate([x[1] for x in st], axis=1))


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def _cpu_share() -> int:
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def covering_rows(nq: int, tile: int = 512, block: int = 32, per_block: int = 2,
                  seed: int = 77) -> np.ndarray:
    """Query rows that reach every `block`-row query block of the partition (per_block
    rows each, at offsets that vary from block to block so that every lane position
    of a block is hit somewhere), the first and last row of every `tile`-row tile,
    and the last row."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b0 in range(0, nq, block):
        n = min(block, nq - b0)
        for j in range(per_block):
            rows.add(b0 + int((b0 // block * 13 + j * (block // per_block) + rng.integers(0, 3)) % n))
    for t0 in range(0, nq, tile):
        rows.add(t0)
        rows.add(min(t0 + tile, nq) - 1)
    rows.add(nq - 1)
    return np.array(sorted(rows), dtype=np.int64)
