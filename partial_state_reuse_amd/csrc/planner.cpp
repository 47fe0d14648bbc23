// Reuse-mask planner: host-only integer arithmetic.
//
// Rules from the DiTango page, Methodology > 1. Anchor-Guided Selection
// Planner: anchor steps recompute every partition; the local partition is
// always computed; every other partition is computed fresh or reuses its
// historical state.  The page prints no selection formula, so the choice is
// one of four fixed schedules (distance radius, k nearest, a Bernoulli(1/2)
// draw from SplitMix64, a linearly ramped radius); a slot holding no state is
// always computed fresh.

#include "planner.h"

namespace dita {

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): the state advances by the
// golden-ratio gamma; each output is the state run through two
// xor-shift-multiply rounds and a final xor-shift.
uint64_t splitmix64_next(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int plan_radius(const dita_plan& plan, int64_t step) {
  const int64_t r0 = plan.radius, r1 = plan.radius_end, t = plan.total_steps;
  if (t <= 1 || step <= 0) return int(r0);
  if (step >= t - 1) return int(r1);
  const int64_t d = t - 1;
  const int64_t n = r0 * d + (r1 - r0) * step;  // in [min(r0,r1)*d, max(r0,r1)*d], >= 0
  return int((2 * n + d) / (2 * d));           // round half up
}

bool plan_valid(const dita_plan& plan) {
  return plan.P >= 1 && plan.P <= DITA_MAX_PARTITIONS && plan.q >= 0 && plan.q < plan.P &&
         plan.policy >= DITA_PLAN_DIST && plan.policy <= DITA_PLAN_RAMP && plan.radius >= 0 &&
         plan.radius_end >= 0 && plan.k_nearest >= 0 && plan.anchor_period >= 0 &&
         plan.total_steps >= 1;
}

static int64_t absdiff(int a, int b) { return a > b ? a - b : b - a; }

void plan_mask(const dita_plan& plan, int64_t step, const uint8_t* valid, uint8_t* reuse) {
  const int P = plan.P, q = plan.q;
  switch (plan.policy) {
    case DITA_PLAN_DIST:
    case DITA_PLAN_RAMP: {
      const int64_t r = plan.policy == DITA_PLAN_DIST ? plan.radius : plan_radius(plan, step);
      for (int p = 0; p < P; ++p) reuse[p] = absdiff(p, q) > r ? 1 : 0;
      break;
    }
    case DITA_PLAN_KNEAREST: {
      // Rank of p in the order (|p - q|, p): the number of partitions before it.
      for (int p = 0; p < P; ++p) {
        int rank = 0;
        for (int o = 0; o < P; ++o) {
          const int64_t dp = absdiff(p, q), dq = absdiff(o, q);
          if (dq < dp || (dq == dp && o < p)) ++rank;
        }
        reuse[p] = rank < plan.k_nearest ? 0 : 1;
      }
      break;
    }
    case DITA_PLAN_RANDOM: {
      uint64_t state = (plan.seed << 32) ^ uint64_t(step);
      for (int p = 0; p < P; ++p) reuse[p] = uint8_t(splitmix64_next(&state) >> 63);
      break;
    }
  }
  reuse[q] = 0;
  if (plan.anchor_period > 0 && step % plan.anchor_period == 0)
    for (int p = 0; p < P; ++p) reuse[p] = 0;
  if (valid)
    for (int p = 0; p < P; ++p)
      if (!valid[p]) reuse[p] = 0;
}

}  // namespace dita
