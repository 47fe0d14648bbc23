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

Section "Dynamic Group Compose" of the same page merges cached states
recursively into coarser groups, cutting memory without recomputation.  Here a
group is a contiguous range of partitions [first, last] whose cached states
have been composed (merged) into one state held in slot ``first``; the other
slots of the range hold nothing of their own any more.  Reading taken where the
page is silent: a group is reused only as a whole -- when every member is
marked reuse -- and otherwise all of its members are recomputed fresh, which
dissolves it back into single-partition slots.  A group's stamp is the oldest
stamp among the states composed into it, and every member carries it.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .attention import State, merge_states, partial_state
from .compress import compact_state


@dataclass
class StateCache:
    """P slots of (O_p, LSE_p) with a valid flag, the step that wrote each, and
    the group (leader slot) each partition belongs to."""

    P: int
    slots: List[Optional[State]] = field(default_factory=list)
    valid: np.ndarray = None
    stamp: np.ndarray = None
    group: np.ndarray = None

    def __post_init__(self):
        if self.P < 1:
            raise ValueError("P must be >= 1")
        self.slots = [None] * self.P
        self.valid = np.zeros(self.P, dtype=np.uint8)
        self.stamp = np.full(self.P, -1, dtype=np.int64)
        self.group = np.arange(self.P, dtype=np.int64)

    def group_range(self, p: int):
        """(first, last) of the group holding partition p."""
        first = int(self.group[p])
        last = first
        while last + 1 < self.P and self.group[last + 1] == first:
            last += 1
        return first, last

    def leaders(self) -> List[int]:
        """First slot of every group (a lone partition is its own group), in order."""
        return [p for p in range(self.P) if self.group[p] == p]

    def live_states(self) -> int:
        """Number of slots that hold a state of their own."""
        return sum(1 for p in self.leaders() if self.valid[p])

    def store(self, p: int, state: State, step: int) -> None:
        if self.group_range(p) != (p, p):
            raise RuntimeError(f"partition {p} belongs to a composed group")
        o, lse = state
        self.slots[p] = (np.array(o, dtype=np.float64), np.array(lse, dtype=np.float64))
        self.valid[p] = 1
        self.stamp[p] = step

    def invalidate(self, p: int = -1) -> None:
        if p < 0:
            idx = range(self.P)
        else:
            first, last = self.group_range(p)
            idx = range(first, last + 1)
        for i in idx:
            self.slots[i] = None
            self.valid[i] = 0
            self.stamp[i] = -1
            self.group[i] = i

    def compact(self, p: int) -> None:
        """Hold group leader p's state in the compact encoding (see compress.py):
        from now on its output is the decoded int8 codes times the row scales,
        its LSE unchanged.  A later store (a fresh state) replaces it."""
        if self.group[p] != p or not self.valid[p]:
            raise RuntimeError(f"partition {p} does not lead a group holding a state")
        self.slots[p] = compact_state(self.slots[p])

    def dissolve(self, first: int) -> None:
        """Forget a group: its members become single, empty slots."""
        _, last = self.group_range(first)
        for i in range(first, last + 1):
            self.slots[i] = None
            self.valid[i] = 0
            self.stamp[i] = -1
            self.group[i] = i

    def compose(self, first: int, last: int) -> None:
        """Merge the cached states of partitions first..last into one group
        state held in slot ``first`` (groups already inside the range are
        merged as the single states they are)."""
        if not (0 <= first <= last < self.P):
            raise ValueError("need 0 <= first <= last < P")
        for p in range(first, last + 1):
            if not self.valid[p]:
                raise RuntimeError(f"partition {p} holds no state")
            a, b = self.group_range(p)
            if a < first or b > last:
                raise ValueError(f"group [{a}, {b}] straddles the range [{first}, {last}]")
        heads = [p for p in range(first, last + 1) if self.group[p] == p]
        state = merge_states([self.slots[p] for p in heads])
        oldest = min(int(self.stamp[p]) for p in heads)
        for p in range(first, last + 1):
            self.slots[p] = None
            self.group[p] = first
            self.valid[p] = 1
            self.stamp[p] = oldest
        self.slots[first] = (state[0], state[1])


def compose_runs(cache: StateCache, reuse: Sequence[int]) -> int:
    """Compose ahead of a step: each maximal run of partitions that ``reuse``
    marks for reuse becomes one group, without the groups that reach outside
    the run (a step with this mask recomputes those whole).  A run of one
    partition, or one that already is a single group, is left alone.
    Returns the number of compositions that merged two or more states.

    Reading taken where the page is silent: the page composes cached states
    into coarser groups but names no rule for which; composing exactly what
    the next step reuses keeps every group reusable whole at that step."""
    reuse = np.asarray(reuse, dtype=np.uint8)
    for p in range(cache.P):
        if reuse[p] and not cache.valid[p]:
            raise RuntimeError(f"partition {p} is marked reuse but its slot is empty")
    runs = []
    p = 0
    while p < cache.P:
        if not reuse[p]:
            p += 1
            continue
        a = p
        while p + 1 < cache.P and reuse[p + 1]:
            p += 1
        b = p
        p += 1
        inside = [i for i in range(a, b + 1)
                  if cache.group_range(i)[0] >= a and cache.group_range(i)[1] <= b]
        if not inside:
            continue
        lo, hi = min(inside), max(inside)
        if lo < hi and cache.group_range(lo) != (lo, hi):
            runs.append((lo, hi))
    merged = 0
    for a, b in runs:
        heads = [i for i in range(a, b + 1) if cache.group[i] == i]
        merged += len(heads) > 1
        cache.compose(a, b)
    return merged


def effective_reuse(cache: StateCache, reuse: Sequence[int]) -> np.ndarray:
    """The mask a step actually applies: a composed group is reused only when
    every member is marked reuse; otherwise all its members are recomputed."""
    reuse = np.asarray(reuse, dtype=np.uint8).copy()
    for first in cache.leaders():
        _, last = cache.group_range(first)
        if last > first and not reuse[first:last + 1].all():
            reuse[first:last + 1] = 0
    return reuse


def attn_step(cache: StateCache, q, k_parts: Sequence, v_parts: Sequence,
              reuse: Sequence[int], step: int, scale: float | None = None):
    """One rank-step: refresh the fresh slots, keep the reused ones, merge all.

    ``reuse[p]`` is 1 to reuse slot p and 0 to compute it fresh.  Groups are
    reused or recomputed whole (``effective_reuse``).  Returns
    ``(O, LSE, n_fresh)`` with n_fresh counting recomputed partitions.  Reusing
    a slot that was never filled raises.
    """
    reuse = np.asarray(reuse, dtype=np.uint8)
    if reuse.shape != (cache.P,) or len(k_parts) != cache.P or len(v_parts) != cache.P:
        raise ValueError("mask, K and V lists must have P entries")
    for p in range(cache.P):
        if reuse[p] and not cache.valid[p]:
            raise RuntimeError(f"partition {p} is marked reuse but its slot is empty")
    reuse = effective_reuse(cache, reuse)
    for first in cache.leaders():
        _, last = cache.group_range(first)
        if last > first and not reuse[first]:
            cache.dissolve(first)
    n_fresh = 0
    for p in range(cache.P):
        if not reuse[p]:
            cache.store(p, partial_state(q, k_parts[p], v_parts[p], scale), step)
            n_fresh += 1
    o, lse = merge_states([cache.slots[p] for p in cache.leaders()])
    return o, lse, n_fresh
