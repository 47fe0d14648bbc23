"""Synthetic workloads: configuration records and seeded input generators.

Shared by the oracle side (tests, CPU baseline) and the GPU side (tests,
benchmark).  Holds no arithmetic of the attention method itself.
"""

from .configs import (
    ORDER,
    POLICY_DIST,
    POLICY_KNEAREST,
    POLICY_RAMP,
    POLICY_RANDOM,
    WORKLOADS,
    Workload,
    get,
    reduced,
)
from .inputs import Inputs, grid_coords, round_bf16, split_parts

__all__ = [
    "ORDER", "WORKLOADS", "Workload", "get", "reduced", "Inputs", "grid_coords",
    "round_bf16", "split_parts", "POLICY_DIST", "POLICY_KNEAREST", "POLICY_RANDOM",
    "POLICY_RAMP",
]
