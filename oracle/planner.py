"""Reuse-mask planner and its integer generator, in plain Python.

Test infrastructure only (see the package docstring).

The DiTango page, Methodology > "1. Anchor-Guided Selection Planner", fixes
three rules that every policy here obeys:

* anchor steps recompute every partition ("Anchor Steps");
* the rank's own (local) partition is always computed ("Online Prediction":
  local state changes are always computed);
* otherwise a partition is either computed fresh or its historical state is
  reused.

The page gives no formula for the choice itself (its error model in w and
delta is not printed), so the policies are the plain deterministic schedules
of the five synthetic workloads: a distance radius, the k nearest partitions,
a Bernoulli(1/2) draw per partition, and a radius that ramps linearly over the
schedule.  A slot that was never filled is always computed fresh.

Mask convention: ``uint8[P]``, 1 = reuse the cached state, 0 = compute fresh.
Everything is integer arithmetic so that an independent implementation can
agree bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

POLICY_DIST = 0      # fresh iff |p - q| <= radius
POLICY_KNEAREST = 1  # fresh iff p is among the k nearest partitions (ties -> lower index)
POLICY_RANDOM = 2    # fresh iff the top bit of a SplitMix64 draw is 0
POLICY_RAMP = 3      # radius ramps from `radius` to `radius_end` over `total_steps`

_MASK64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014; the 64-bit finaliser of Vigna's public
    splitmix64 reference): the state advances by the golden-ratio gamma
    0x9E3779B97F4A7C15 and each output is the state passed through two
    xor-shift-multiply rounds and a final xor-shift."""

    GAMMA = 0x9E3779B97F4A7C15

    def __init__(self, seed: int):
        self.state = seed & _MASK64

    def next(self) -> int:
        self.state = (self.state + self.GAMMA) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)


@dataclass(frozen=True)
class Plan:
    """Planner parameters; mirrors the library's plan struct field for field."""

    P: int
    q: int
    policy: int = POLICY_DIST
    radius: int = 0
    radius_end: int = 0
    k_nearest: int = 1
    anchor_period: int = 0     # 0: no periodic anchors
    total_steps: int = 1
    seed: int = 0


def radius_at(plan: Plan, step: int) -> int:
    """Radius of the ramp policy at ``step``: round-half-up of the linear
    interpolation from ``radius`` (step 0) to ``radius_end`` (step
    total_steps-1), computed in integers; clamped outside the schedule."""
    r0, r1, t = plan.radius, plan.radius_end, plan.total_steps
    if t <= 1 or step <= 0:
        return r0
    if step >= t - 1:
        return r1
    d = t - 1
    n = r0 * d + (r1 - r0) * step     # between r0*d and r1*d, both >= 0
    return (2 * n + d) // (2 * d)


def plan_mask(plan: Plan, step: int, valid: Optional[Sequence[int]] = None) -> np.ndarray:
    """Reuse mask for ``step`` (1 = reuse, 0 = fresh).

    ``valid`` (optional, length P) marks which cache slots hold a state; an
    invalid slot can only be computed fresh.
    """
    P, q = plan.P, plan.q
    if not (1 <= P <= 64) or not (0 <= q < P) or step < 0:
        raise ValueError("need 1 <= P <= 64, 0 <= q < P, step >= 0")
    reuse = np.zeros(P, dtype=np.uint8)
    if plan.policy == POLICY_DIST or plan.policy == POLICY_RAMP:
        r = plan.radius if plan.policy == POLICY_DIST else radius_at(plan, step)
        for p in range(P):
            reuse[p] = 1 if abs(p - q) > r else 0
    elif plan.policy == POLICY_KNEAREST:
        order = sorted(range(P), key=lambda p: (abs(p - q), p))
        near = set(order[: max(plan.k_nearest, 0)])
        for p in range(P):
            reuse[p] = 0 if p in near else 1
    elif plan.policy == POLICY_RANDOM:
        gen = SplitMix64(((plan.seed << 32) ^ step) & _MASK64)
        for p in range(P):
            draw = gen.next()            # drawn for every p, the local one included
            reuse[p] = draw >> 63
    else:
        raise ValueError(f"unknown policy {plan.policy}")
    # Overrides: the local partition, anchor steps and never-filled slots are fresh.
    reuse[q] = 0
    if plan.anchor_period > 0 and step % plan.anchor_period == 0:
        reuse[:] = 0
    if valid is not None:
        valid = np.asarray(valid)
        if valid.shape != (P,):
            raise ValueError("valid must have P entries")
        reuse[valid == 0] = 0
    return reuse
