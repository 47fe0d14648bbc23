"""Per-partition state cache and one compute-or-reuse rank-step, float64.

Test infrastructure only (see the package docstring).

The DiTango page, Methodology > 2. State-Centric Parallel Runtime > "State
Composition", caches composed attention states instead of raw K/V; section
"1. Anchor-Guided Selection Planner" decides per partition whether a state is
computed fresh or a historical one is reused.  A rank-step therefore:

1. for every partition p marked fresh: computes its partial state from the
   current K_p, V_p and stores it in slot p, stamped with the step index;
2. for every partition p marked reuse: takes slot p as it is (it must have
   been filled before);
3. merges all P slots into the rank's output.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .attention import State, merge_states, partial_state


@dataclass
class StateCache:
    """P slots of (O_p, LSE_p) with a valid flag and the step that wrote each."""

    P: int
    slots: List[Optional[State]] = field(default_factory=list)
    valid: np.ndarray = None
    stamp: np.ndarray = None

    def __post_init__(self):
        if self.P < 1:
            raise ValueError("P must be >= 1")
        self.slots = [None] * self.P
        self.valid = np.zeros(self.P, dtype=np.uint8)
        self.stamp = np.full(self.P, -1, dtype=np.int64)

    def store(self, p: int, state: State, step: int) -> None:
        o, lse = state
        self.slots[p] = (np.array(o, dtype=np.float64), np.array(lse, dtype=np.float64))
        self.valid[p] = 1
        self.stamp[p] = step

    def invalidate(self, p: int = -1) -> None:
        idx = range(self.P) if p < 0 else [p]
        for i in idx:
            self.slots[i] = None
            self.valid[i] = 0
            self.stamp[i] = -1


def attn_step(cache: StateCache, q, k_parts: Sequence, v_parts: Sequence,
              reuse: Sequence[int], step: int, scale: float | None = None):
    """One rank-step: refresh the fresh slots, keep the reused ones, merge all.

    ``reuse[p]`` is 1 to reuse slot p and 0 to compute it fresh.  Returns
    ``(O, LSE, n_fresh)``.  Reusing a slot that was never filled raises.
    """
    reuse = np.asarray(reuse, dtype=np.uint8)
    if reuse.shape != (cache.P,) or len(k_parts) != cache.P or len(v_parts) != cache.P:
        raise ValueError("mask, K and V lists must have P entries")
    for p in range(cache.P):
        if reuse[p] and not cache.valid[p]:
            raise RuntimeError(f"partition {p} is marked reuse but its slot is empty")
    n_fresh = 0
    for p in range(cache.P):
        if not reuse[p]:
            cache.store(p, partial_state(q, k_parts[p], v_parts[p], scale), step)
            n_fresh += 1
    o, lse = merge_states(cache.slots)
    return o, lse, n_fresh
