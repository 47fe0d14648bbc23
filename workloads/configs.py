"""The five synthetic workloads: shapes, dtypes, mask schedules, step counts.

Pure data.  Both the oracle side and the GPU side read these descriptions;
neither side's arithmetic lives here.

Shapes follow video-DiT attention as the DiTango page describes its targets
(720p video generation with Wan2.1 / HunyuanVideo, "Problem Statement" and
"Experimental Results"): a t-major (frame, row, column) token grid is split
into P equal, contiguous context partitions; one rank owns partition ``q`` as
its queries and attends to all P partitions.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional, Tuple

# Mask policies (same numbering as the library's plan struct and the oracle).
POLICY_DIST = 0
POLICY_KNEAREST = 1
POLICY_RANDOM = 2
POLICY_RAMP = 3


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    grid: Tuple[int, int, int]      # (frames, rows, cols); N = product
    P: int                          # context partitions
    dtype: str                      # "f32" or "bf16"
    values: str                     # "gauss": N(0,1); "fourier": RFF on the grid + noise
    q_part: int = 0                 # the rank's query partition
    # mask schedule
    policy: int = POLICY_DIST
    radius: int = 0
    radius_end: int = 0
    k_nearest: int = 1
    anchor_period: int = 0
    mask_seed: int = 1
    # step schedule
    steps: int = 2                  # rank-steps in the schedule (including the cache fill)
    single_step: bool = True        # step 0 fills the cache from perturbed K/V, step 1 is measured
    perturb: float = 0.05           # cache-fill perturbation (single-step schedules)
    drift: float = 0.02             # per-step K/V drift (multi-step schedules)
    noise: float = 0.5              # noise added to the Fourier features

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def Nk(self) -> int:
        if self.N % self.P:
            raise ValueError("N must split into P equal partitions")
        return self.N // self.P

    @property
    def Nq(self) -> int:
        return self.Nk

    def part_range(self, p: int) -> Tuple[int, int]:
        return p * self.Nk, (p + 1) * self.Nk

    def plan_fields(self) -> Dict[str, int]:
        """Keyword arguments for the planner's plan record."""
        return dict(P=self.P, q=self.q_part, policy=self.policy, radius=self.radius,
                    radius_end=self.radius_end, k_nearest=self.k_nearest,
                    anchor_period=self.anchor_period, total_steps=self.steps,
                    seed=self.mask_seed)

    def block_flops(self) -> int:
        """Matrix-product flops of one fresh (query partition, KV partition) block:
        2*Nq*Nk*D for Q K^T plus 2*Nq*Nk*D for P V, per batch and head."""
        return 4 * self.B * self.H * self.Nq * self.Nk * self.D

    def state_bytes(self) -> int:
        """Bytes of one attention state: O in the workload dtype plus fp32 LSE."""
        esz = 4 if self.dtype == "f32" else 2
        return self.B * self.H * self.Nq * (self.D * esz + 4)

    def merge_bytes(self) -> int:
        """Algorithmic HBM bytes of one P-way merge: read P states, write one."""
        return (self.P + 1) * self.state_bytes()


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 case: sequence 1024 in 4 partitions of 256, queries = partition 0,
    # N(0,1) values, recompute partitions at distance <= 1.
    "tiny_f32": Workload(name="tiny_f32", B=1, H=2, D=64, grid=(4, 16, 16), P=4,
                         dtype="f32", values="gauss", policy=POLICY_DIST, radius=1),
    # 16k tokens on a 16x32x32 grid, 8 partitions of 2048, 50% random reuse.
    "dit16k_bf16": Workload(name="dit16k_bf16", B=1, H=12, D=64, grid=(16, 32, 32), P=8,
                            dtype="bf16", values="fourier", policy=POLICY_RANDOM),
    # 21 latent frames x 30x52 patches (832x480 at stride 16), 8 partitions of 4095;
    # the 2 nearest partitions (the local one included) are fresh.
    "dit32k_bf16": Workload(name="dit32k_bf16", B=1, H=40, D=128, grid=(21, 30, 52), P=8,
                            dtype="bf16", values="fourier", policy=POLICY_KNEAREST,
                            k_nearest=2),
    # 21 frames x 45x80 patches (720p at stride 16), 16 partitions of 4725; radius 2,
    # a full refresh (anchor) every 5th step, 10 steps.
    "dit75k_bf16": Workload(name="dit75k_bf16", B=1, H=40, D=128, grid=(21, 45, 80), P=16,
                            dtype="bf16", values="fourier", policy=POLICY_DIST, radius=2,
                            anchor_period=5, steps=10, single_step=False),
    # Same shape over 50 denoising steps; the radius ramps 8 -> 1; only step 0 is cold.
    "dit75k_ramp50": Workload(name="dit75k_ramp50", B=1, H=40, D=128, grid=(21, 45, 80), P=16,
                              dtype="bf16", values="fourier", policy=POLICY_RAMP, radius=8,
                              radius_end=1, steps=50, single_step=False),
}

# Order of the five workloads (tiny fp32 first, the 50-step schedule last).
ORDER = ["tiny_f32", "dit16k_bf16", "dit32k_bf16", "dit75k_bf16", "dit75k_ramp50"]


def get(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return replace(wl, **overrides) if overrides else wl


def reduced(name: str, H: Optional[int] = None, grid: Optional[Tuple[int, int, int]] = None,
            **overrides) -> Workload:
    """A smaller copy of a workload (fewer heads and/or a smaller grid) for fast tests."""
    wl = WORKLOADS[name]
    kw = dict(overrides)
    if H is not None:
        kw["H"] = H
    if grid is not None:
        kw["grid"] = grid
    return replace(wl, name=wl.name + "_reduced", **kw)
