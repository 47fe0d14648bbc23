// Host-only reuse-mask planner (no HIP dependency).
#pragma once

#include <cstdint>

#include "../../include/dita.h"

namespace dita {

uint64_t splitmix64_next(uint64_t* state);
int plan_radius(const dita_plan& plan, int64_t step);
bool plan_valid(const dita_plan& plan);
// valid: P bytes or nullptr; reuse: P bytes written.
void plan_mask(const dita_plan& plan, int64_t step, const uint8_t* valid, uint8_t* reuse);
// Error-guided planner: P bytes of reuse and P doubles of estimated error written.
void error_plan_mask(const dita_planner& pl, int64_t step, const uint8_t* valid,
                     const int64_t* stamp, uint8_t* reuse, double* err);

}  // namespace dita
