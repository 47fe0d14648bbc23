// Error-guided, group-wise reuse planner (host only, float64).
//
// The DiTango page, Methodology > 1. Anchor-Guided Selection Planner, names the
// parts without a formula: the error of reusing a state depends on the
// partition's importance w and on the temporal growth delta (Error Modeling);
// anchor steps recompute everything and refresh w (Anchor Steps); between
// anchors the change of the always-computed local state predicts the change of
// the remote ones (Online Prediction); decisions are taken per group of
// spatially adjacent partitions (Group-wise Strategy).
//
// This planner:
//   err_p  = w_p * sum_{t = stamp_p + 1 .. s} delta~_t, where delta~_t is the
//            change observed at the latest step <= min(t, s - 1), or the
//            earliest observed change when no observation precedes t;
//   groups = contiguous blocks of group_size partition indices; a group's
//            error is the sum of its members' (the local partition excluded);
//   choice = groups in increasing (error, index) order are reused while the
//            running error stays within the budget; the rest are computed.
// Everything is fresh on an anchor step, before weights are set and before a
// change has been observed; the local partition is always fresh; a group
// holding an invalid slot, or (fresh_weight > 0) a partition of weight >=
// fresh_weight, is fresh.  All sums run in ascending index order in
// float64, so an implementation that follows the same order agrees bit for bit.

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "../../include/dita.h"
#include "planner.h"

struct dita_planner {
  dita_error_plan plan;
  bool has_weights;
  double w[DITA_MAX_PARTITIONS];
  std::vector<std::pair<int64_t, double>> seen;  // (step, change), ascending steps
};

namespace dita {

namespace {

bool error_plan_valid(const dita_error_plan& p) {
  return p.P >= 1 && p.P <= DITA_MAX_PARTITIONS && p.q >= 0 && p.q < p.P && p.group_size >= 1 &&
         p.anchor_period >= 0 && !std::isnan(p.budget) && p.budget >= 0.0 &&
         !std::isnan(p.fresh_weight) && p.fresh_weight >= 0.0;
}

// delta~_t for planning `step`: observations after step - 1 are not known yet.
double change_at(const dita_planner& pl, int64_t t, int64_t step) {
  const std::pair<int64_t, double>* latest = nullptr;
  for (const auto& o : pl.seen) {
    if (o.first > step - 1) break;
    if (o.first <= t) latest = &o;
  }
  return latest ? latest->second : pl.seen.front().second;
}

}  // namespace

void error_plan_mask(const dita_planner& pl, int64_t step, const uint8_t* valid,
                     const int64_t* stamp, uint8_t* reuse, double* err) {
  const int P = pl.plan.P, q = pl.plan.q, g = pl.plan.group_size;
  for (int p = 0; p < P; ++p) {
    reuse[p] = 0;
    err[p] = 0.0;
  }
  const bool anchor = pl.plan.anchor_period > 0 && step % pl.plan.anchor_period == 0;
  const bool observed = !pl.seen.empty() && pl.seen.front().first <= step - 1;
  if (anchor || !pl.has_weights || !observed) return;
  for (int p = 0; p < P; ++p) {
    if (p == q || !valid[p]) continue;
    double growth = 0.0;
    for (int64_t t = stamp[p] + 1; t <= step; ++t) growth += change_at(pl, t, step);
    err[p] = pl.w[p] * growth;
  }
  struct Cand {
    double e;
    int j;
  };
  std::vector<Cand> cands;
  for (int j = 0, a = 0; a < P; ++j, a += g) {
    const int b = std::min(a + g, P) - 1;
    bool any = false, ok = true;
    double e = 0.0;
    for (int p = a; p <= b; ++p) {
      if (p == q) continue;
      any = true;
      ok = ok && valid[p];
      if (pl.plan.fresh_weight > 0.0 && pl.w[p] >= pl.plan.fresh_weight) ok = false;
      e += err[p];
    }
    if (any && ok) cands.push_back({e, j});
  }
  std::stable_sort(cands.begin(), cands.end(), [](const Cand& x, const Cand& y) {
    return x.e < y.e || (x.e == y.e && x.j < y.j);
  });
  double spent = 0.0;
  for (const Cand& c : cands) {
    if (spent + c.e > pl.plan.budget) break;
    spent += c.e;
    const int a = c.j * g, b = std::min(a + g, P) - 1;
    for (int p = a; p <= b; ++p)
      if (p != q) reuse[p] = 1;
  }
}

}  // namespace dita

extern "C" {

int dita_planner_create(dita_planner** out, const dita_error_plan* plan) {
  if (!out || !plan || !dita::error_plan_valid(*plan)) return DITA_ERR_ARG;
  dita_planner* pl = new (std::nothrow) dita_planner;
  if (!pl) return DITA_ERR_ARG;
  pl->plan = *plan;
  pl->has_weights = false;
  for (double& x : pl->w) x = 0.0;
  *out = pl;
  return DITA_OK;
}

int dita_planner_free(dita_planner* planner) {
  delete planner;
  return DITA_OK;
}

int dita_planner_set_weights(dita_planner* planner, const double* w) {
  if (!planner || !w) return DITA_ERR_ARG;
  for (int p = 0; p < planner->plan.P; ++p)
    if (!std::isfinite(w[p]) || w[p] < 0.0) return DITA_ERR_ARG;
  for (int p = 0; p < planner->plan.P; ++p) planner->w[p] = w[p];
  planner->has_weights = true;
  return DITA_OK;
}

int dita_planner_observe(dita_planner* planner, int64_t step, double change) {
  if (!planner || step < 0 || !std::isfinite(change) || change < 0.0) return DITA_ERR_ARG;
  auto& s = planner->seen;
  auto it = std::lower_bound(s.begin(), s.end(), step,
                             [](const std::pair<int64_t, double>& o, int64_t v) { return o.first < v; });
  if (it != s.end() && it->first == step)
    it->second = change;
  else
    s.insert(it, {step, change});
  return DITA_OK;
}

int dita_planner_mask(const dita_planner* planner, int64_t step, const uint8_t* valid,
                      const int64_t* stamp, uint8_t* reuse_out, double* err_out) {
  if (!planner || !valid || !stamp || !reuse_out || step < 0) return DITA_ERR_ARG;
  const int P = planner->plan.P;
  for (int p = 0; p < P; ++p)
    if (valid[p] > 1 || (valid[p] && (stamp[p] < 0 || stamp[p] > step))) return DITA_ERR_ARG;
  double err[DITA_MAX_PARTITIONS];
  dita::error_plan_mask(*planner, step, valid, stamp, reuse_out, err);
  if (err_out)
    for (int p = 0; p < P; ++p) err_out[p] = err[p];
  return DITA_OK;
}

}  // extern "C"
