"""Reference oracle for selective attention-state reuse -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 CPU statement of what the hot path
computes.  It exists so that the tests, the smoke check and the CPU-baseline
leg of the benchmark can check the HIP library against something obviously
correct.  Nothing in the product path (the ``partial_state_reuse_amd``
package and its HIP/C++ sources) imports, calls or links it, and it imports
nothing from there.

Source of the method: the web page "DiTango: Cost-Effective Parallel
Diffusion Generation with Selective Attention State Reuse" (gist.science,
paper 2607.15650), section "Methodology":

* "1. Anchor-Guided Selection Planner" (anchor steps, the always-computed
  local partition, the compute-or-reuse decision per partition), and
* "2. State-Centric Parallel Runtime" -> "State Composition" (an attention
  state is an output plus its log-sum-exp; states compose associatively and
  commutatively; composed states are cached instead of raw K/V) and "Dynamic
  Group Compose" (cached states merged recursively into coarser groups).

Modules
-------
attention  partial attention state, LSE merge, full attention (float64).
cache      the per-partition state cache, group composition and one
           compute-or-reuse rank-step.
planner    the reuse-mask planner and its SplitMix64 integer generator.
error_planner  contribution weights, local state change and the group-wise,
           error-budgeted planner ("Error Modeling", "Online Prediction",
           "Group-wise Strategy" of the planner section).
compress   the compact (int8 codes, per-row scale) encoding of a cached
           state ("Significance and Claims": memory held by cached states,
           cache compression as future work).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, textbook/library routines it does not itself call (scipy's
logsumexp, torch's CPU scaled-dot-product attention), brute-force scalar
loops on tiny inputs, and published generator outputs.  No function is
"parity unpinned" except the error-curve reporting of the 50-step schedule,
which the pages give no numbers for.
"""

from .attention import full_attention, merge_states, partial_state, softmax_scale
from .cache import StateCache, attn_step, compose_runs, effective_reuse
from .compress import compact_state, decode_rows, encode_rows
from .error_planner import ErrorPlanner, contributions, state_change
from .planner import (
    POLICY_DIST,
    POLICY_KNEAREST,
    POLICY_RAMP,
    POLICY_RANDOM,
    Plan,
    SplitMix64,
    plan_mask,
    radius_at,
)

__all__ = [
    "softmax_scale",
    "partial_state",
    "merge_states",
    "full_attention",
    "StateCache",
    "attn_step",
    "effective_reuse",
    "compose_runs",
    "encode_rows",
    "decode_rows",
    "compact_state",
    "ErrorPlanner",
    "contributions",
    "state_change",
    "Plan",
    "SplitMix64",
    "plan_mask",
    "radius_at",
    "POLICY_DIST",
    "POLICY_KNEAREST",
    "POLICY_RANDOM",
    "POLICY_RAMP",
]
