"""Error-guided reuse planner: contribution weights, local state change, and the
group-wise compute-or-reuse choice, in plain Python (float64).

Test infrastructure only (see the package docstring).

The DiTango page, Methodology > "1. Anchor-Guided Selection Planner", names
the parts of its planner without printing a formula:

* Error Modeling -- the error of reusing a partition's attention state is a
  function of the partition's importance w and of the temporal growth delta;
* Anchor Steps -- periodic steps recompute everything, reset the error and
  refresh the importance weights;
* Online Prediction -- between anchors, the change of the local state (which
  is always computed) stands in for the change of every remote state;
* Group-wise Strategy -- spatially adjacent partitions form groups and the
  decision is taken per group: high-contribution groups are computed,
  low-contribution ones reused.

Readings taken here (the plainest ones the page supports):

* importance w_p = the mean, over all query rows, of partition p's softmax
  weight in the merged output, exp(LSE_p - LSE) (these sum to 1 per row);
  measured at an anchor step, where every state is fresh;
* growth delta_t = relative Frobenius change of the local partition's output
  state between steps t-1 and t, ||O_q(t) - O_q(t-1)|| / ||O_q(t-1)||;
* the estimated error of reusing p at step s is w_p times the growth
  accumulated since p was computed (its stamp), sum over t in (stamp_p, s] of
  delta_t; a step not observed takes the latest observed delta before it (the
  prediction), or the earliest observed one if it precedes every observation;
* groups are the contiguous blocks of ``group_size`` partition indices; a
  group's error is the sum of its members' (the local partition excluded --
  it is always computed); groups are taken for reuse in increasing order of
  error (ties by index) while the running sum of reused error stays within
  ``budget``; every other group is computed;
* forced fresh: the local partition; every partition on an anchor step, when
  no weights are set yet, or when no change has been observed yet; every
  member of a group holding a slot without a state; and, when
  ``fresh_weight`` > 0, every member of a group holding a partition whose
  weight is at least ``fresh_weight`` (the page: high-contribution partitions
  are computed).
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def contributions(lse_parts: Sequence, lse) -> np.ndarray:
    """w_p = mean over rows of exp(LSE_p - LSE).  Rows whose merged LSE is -inf
    contribute 0 to every partition (they have no weight to share)."""
    lse = np.asarray(lse, dtype=np.float64).reshape(-1)
    out = np.zeros(len(lse_parts))
    finite = np.isfinite(lse)
    for p, lp in enumerate(lse_parts):
        lp = np.asarray(lp, dtype=np.float64).reshape(-1)
        w = np.zeros_like(lse)
        ok = finite & np.isfinite(lp)
        w[ok] = np.exp(lp[ok] - lse[ok])
        out[p] = float(np.sum(w)) / lse.size
    return out


def state_change(o_new, o_prev) -> float:
    """||o_new - o_prev||_F / ||o_prev||_F (0 when both are 0, inf when only
    o_prev is 0)."""
    a = np.asarray(o_new, dtype=np.float64)
    b = np.asarray(o_prev, dtype=np.float64)
    num = math.sqrt(float(np.sum((a - b) ** 2)))
    den = math.sqrt(float(np.sum(b ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


class ErrorPlanner:
    """Group-wise, error-budgeted compute-or-reuse planner (readings above)."""

    def __init__(self, P: int, q: int, group_size: int, budget: float, anchor_period: int = 0,
                 fresh_weight: float = 0.0):
        if not (1 <= P <= 64 and 0 <= q < P and group_size >= 1 and budget >= 0.0
                and anchor_period >= 0 and fresh_weight >= 0.0):
            raise ValueError("bad planner parameters")
        self.P, self.q, self.g = P, q, group_size
        self.budget = float(budget)
        self.anchor_period = anchor_period
        self.fresh_weight = float(fresh_weight)
        self.weights: Optional[List[float]] = None
        self.delta: Dict[int, float] = {}

    def set_weights(self, w: Sequence[float]) -> None:
        if len(w) != self.P or not all(math.isfinite(float(x)) and float(x) >= 0.0 for x in w):
            raise ValueError("need P finite, non-negative weights")
        self.weights = [float(x) for x in w]

    def observe(self, step: int, delta: float) -> None:
        """Record the local state change measured at ``step`` (a later call for
        the same step replaces it)."""
        if step < 0 or not (math.isfinite(float(delta)) and float(delta) >= 0.0):
            raise ValueError("need step >= 0 and a finite, non-negative change")
        self.delta[int(step)] = float(delta)

    def _delta_at(self, t: int, step: int) -> float:
        seen = sorted(u for u in self.delta if u <= step - 1)
        before = [u for u in seen if u <= t]
        return self.delta[before[-1]] if before else self.delta[seen[0]]

    def groups(self) -> List[Tuple[int, int]]:
        return [(a, min(a + self.g, self.P) - 1) for a in range(0, self.P, self.g)]

    def mask(self, step: int, valid: Sequence[int], stamp: Sequence[int]):
        """(reuse uint8[P], estimated error float64[P]) for ``step``."""
        P, q = self.P, self.q
        reuse = np.zeros(P, dtype=np.uint8)
        err = np.zeros(P)
        anchor = self.anchor_period > 0 and step % self.anchor_period == 0
        observed = any(u <= step - 1 for u in self.delta)
        if anchor or self.weights is None or not observed:
            return reuse, err
        for p in range(P):
            if p == q or not valid[p]:
                continue
            growth = 0.0
            for t in range(int(stamp[p]) + 1, step + 1):
                growth += self._delta_at(t, step)
            err[p] = self.weights[p] * growth
        candidates = []
        for j, (a, b) in enumerate(self.groups()):
            members = [p for p in range(a, b + 1) if p != q]
            if not members or not all(valid[p] for p in members):
                continue
            if self.fresh_weight > 0.0 and any(self.weights[p] >= self.fresh_weight for p in members):
                continue
            e = 0.0
            for p in members:
                e += err[p]
            candidates.append((e, j, members))
        candidates.sort(key=lambda c: (c[0], c[1]))
        spent = 0.0
        for e, _, members in candidates:
            if spent + e > self.budget:
                break
            spent += e
            for p in members:
                reuse[p] = 1
        return reuse, err
