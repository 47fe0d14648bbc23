"""Seeded synthetic Q/K/V for the workloads, shared by the oracle side and the GPU side.

Holds no arithmetic of the method (no scores, softmax, states or merges):
only the recipe that draws the inputs (below) and the round-to-nearest-even
narrowing that both sides must see identically.

Recipe
------
* Token n of the t-major grid sits at x = (t, h, w) with n = (t*Hg + h)*Wg + w.
* "gauss": every Q/K/V entry is N(0, 1).
* "fourier": per (batch, head) draw Omega[f, a] ~ N(0, 1/l_a^2), l = (2, 4, 4)
  grid units, and phases b_f ~ U[0, 2 pi); phi(x)_f = sqrt(2/D) cos(Omega_f . x + b_f)
  (random Fourier features of a Gaussian kernel, so phi(x).phi(y) falls with
  distance).  Q and K share (Omega, b) within a head, V has its own:
      Q = a_qk phi(x) + noise * N(0,1),  K likewise,  V = phi_V(x) + noise * N(0,1),
  with a_qk = sqrt(8 sqrt(D)) so that scaled scores of nearby tokens reach ~8.
* Single-step schedules: step 0 fills the cache from K + perturb*N(0,1) and
  V + perturb*N(0,1); step 1 uses K, V.
* Multi-step schedules: K^(s+1) = K^(s) + drift*N(0,1), the same for V; Q fixed.
* bf16 workloads: the float32 masters are rounded to bf16 (nearest-even) once
  per step; both sides consume exactly those values (carried as float32 here).

Random streams are independent per (kind, batch, head, step) through
``numpy.random.SeedSequence(seed, spawn_key=...)``, so any head subset can be
regenerated on its own.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .configs import Workload

LENGTH_SCALES = (2.0, 4.0, 4.0)

_FEAT_QK, _FEAT_V, _NOISE_Q, _NOISE_K, _NOISE_V, _PERT_K, _PERT_V, _DRIFT_K, _DRIFT_V = range(9)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 carrying the bf16 values exactly.  Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(seed: int, kind: int, b: int, h: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(kind, b, h, step)))


def grid_coords(grid: Tuple[int, int, int]) -> np.ndarray:
    """[N, 3] float64 (t, h, w) coordinates in t-major token order."""
    t, h, w = grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    return np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1).astype(np.float64)


def _features(rng: np.random.Generator, coords: np.ndarray, D: int) -> np.ndarray:
    """[N, D] float32 random Fourier features; the phase is taken in float64, the cosine in float32."""
    omega = rng.standard_normal((D, 3)) / np.asarray(LENGTH_SCALES)[None, :]
    phase = rng.uniform(0.0, 2.0 * math.pi, size=D)
    arg = (coords @ omega.T + phase[None, :]).astype(np.float32)
    np.cos(arg, out=arg)
    arg *= np.float32(math.sqrt(2.0 / D))
    return arg


def _workers(n_jobs: int) -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(n_jobs, cores, 16))


class Inputs:
    """Q and per-step K/V of one workload for a subset of heads.

    ``q`` is [B, len(heads), Nq, D]; ``kv(step)`` returns (K, V), each
    [B, len(heads), N, D], partition p being tokens [p*Nk, (p+1)*Nk).  All
    arrays are float32 holding values exactly representable in the workload
    dtype.  Steps must be requested in non-decreasing order (``reset`` goes
    back to step 0).
    """

    def __init__(self, wl: Workload, seed: int = 0, heads: Optional[Sequence[int]] = None):
        self.wl = wl
        self.seed = seed
        self.heads: List[int] = list(range(wl.H)) if heads is None else [int(h) for h in heads]
        self._jobs = [(b, hi, h) for b in range(wl.B) for hi, h in enumerate(self.heads)]
        nh = len(self.heads)
        self.q = np.empty((wl.B, nh, wl.Nq, wl.D), np.float32)
        self._k0 = np.empty((wl.B, nh, wl.N, wl.D), np.float32)
        self._v0 = np.empty_like(self._k0)
        self._parallel(self._gen_base)
        self.q = self._narrow(self.q)
        self.reset()

    # -- generation ---------------------------------------------------------
    def _parallel(self, fn) -> None:
        if len(self._jobs) == 1:
            fn(*self._jobs[0])
            return
        with ThreadPoolExecutor(_workers(len(self._jobs))) as ex:
            list(ex.map(lambda j: fn(*j), self._jobs))

    def _gen_base(self, b: int, hi: int, h: int) -> None:
        wl = self.wl
        q0, q1 = wl.part_range(wl.q_part)
        if wl.values == "gauss":
            self.q[b, hi] = _rng(self.seed, _NOISE_Q, b, h).standard_normal((wl.Nq, wl.D), np.float32)
            self._k0[b, hi] = _rng(self.seed, _NOISE_K, b, h).standard_normal((wl.N, wl.D), np.float32)
            self._v0[b, hi] = _rng(self.seed, _NOISE_V, b, h).standard_normal((wl.N, wl.D), np.float32)
            return
        coords = grid_coords(wl.grid)
        a_qk = np.float32(math.sqrt(8.0 * math.sqrt(wl.D)))
        nz = np.float32(wl.noise)
        phi = _features(_rng(self.seed, _FEAT_QK, b, h), coords, wl.D)
        phi *= a_qk
        q = self.q[b, hi]
        q[...] = phi[q0:q1]
        q += nz * _rng(self.seed, _NOISE_Q, b, h).standard_normal((wl.Nq, wl.D), np.float32)
        k = self._k0[b, hi]
        k[...] = phi
        del phi
        k += nz * _rng(self.seed, _NOISE_K, b, h).standard_normal((wl.N, wl.D), np.float32)
        v = self._v0[b, hi]
        v[...] = _features(_rng(self.seed, _FEAT_V, b, h), coords, wl.D)
        v += nz * _rng(self.seed, _NOISE_V, b, h).standard_normal((wl.N, wl.D), np.float32)

    def _narrow(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.wl.dtype == "bf16" else x

    def reset(self) -> None:
        self._step = 0
        self._k = self._k0.copy()
        self._v = self._v0.copy()

    def _add_noise(self, kind_k: int, kind_v: int, scale: float, step: int,
                   k: np.ndarray, v: np.ndarray) -> None:
        sc = np.float32(scale)

        def job(b, hi, h):
            for x, kind in ((k, kind_k), (v, kind_v)):
                e = _rng(self.seed, kind, b, h, step).standard_normal(x.shape[2:], np.float32)
                e *= sc
                x[b, hi] += e
        self._parallel(job)

    def kv(self, step: int) -> Tuple[np.ndarray, np.ndarray]:
        wl = self.wl
        if step < 0:
            raise ValueError("step must be >= 0")
        if wl.single_step:
            if step == 0:
                k, v = self._k0.copy(), self._v0.copy()
                self._add_noise(_PERT_K, _PERT_V, wl.perturb, 0, k, v)
                return self._narrow_pair(k, v)
            return self._narrow_pair(self._k0, self._v0)
        if step < self._step:
            self.reset()
        while self._step < step:
            self._add_noise(_DRIFT_K, _DRIFT_V, wl.drift, self._step, self._k, self._v)
            self._step += 1
        return self._narrow_pair(self._k, self._v)

    def _narrow_pair(self, k, v):
        if self.wl.dtype != "bf16":
            return k.copy(), v.copy()
        out = [np.empty_like(k), np.empty_like(v)]

        def job(b, hi, h):
            out[0][b, hi] = round_bf16(k[b, hi])
            out[1][b, hi] = round_bf16(v[b, hi])
        self._parallel(job)
        return out[0], out[1]


def split_parts(x: np.ndarray, wl: Workload) -> List[np.ndarray]:
    """Views of the P context partitions of a [B, H, N, D] array."""
    return [x[..., slice(*wl.part_range(p)), :] for p in range(wl.P)]
