// Query-tile layouts of an attention launch: how the query rows of every
// (head, block) pair are cut into 512-row and 256-row tiles, and in which
// order the tiles are dispatched.
//
// A launch runs its workgroups (one per compute unit at a time) in rounds; a
// 256-row tile takes about kSmallTileCost of a 512-row tile's time.  The
// staged layout dispatches every 512-row tile first and every 256-row tile
// after them, and sizes the two sets so that the 512-row tiles fill whole
// rounds: pairs [0, stage_a) have nb 512-row and ns_a 256-row tiles, the others
// nb - 1 512-row tiles and ns_b = the 256-row tiles that cover the 512 rows
// more (ns_a + 2 when the pair has rows past its nb 512-row tiles).
//
// Every function is constexpr, so it serves the host planner, the kernel's
// decode and the CPU tests alike.
#pragma once

#include <cstdint>

namespace dita {

// Time of a 256-row tile relative to a 512-row tile over the same keys
// (measured on one MI355X, 4725 keys per head, D = 128).
constexpr double kSmallTileCost = 0.61;

// Estimated finishing time, in 512-row tile times, of nb 512-row tiles and ns
// 256-row tiles (cost c1 each) on `cus` compute units that each run one
// workgroup at a time and take the next tile when free, with the 256-row tiles
// dispatched after all 512-row tiles.
constexpr double estimated_makespan(int64_t nb, int64_t ns, int cus, double c1) {
  const int64_t r = nb / cus, rem = nb % cus;
  const double big_end = double(r + (rem ? 1 : 0));
  if (ns == 0) return big_end;
  // cus - rem units are free at time r, rem at r + 1; each then runs small
  // tiles back to back.  Hand out the small tiles in order of start time.
  int64_t left = ns, ma = 0, mb = 0;
  double last_start = 0.0;
  while (left > 0) {
    const double ta = double(r) + double(ma) * c1, tb = double(r + 1) + double(mb) * c1;
    if (cus - rem > 0 && (rem == 0 || ta <= tb)) {
      left -= cus - rem;
      last_start = ta;
      ++ma;
    } else {
      left -= rem;
      last_start = tb;
      ++mb;
    }
  }
  const double end = last_start + c1;
  return end > big_end ? end : big_end;
}

struct StagedLayout {
  int nb;       // 512-row tiles of pairs [0, stage_a); the others have nb - 1
  int ns_a;     // 256-row tiles of pairs [0, stage_a)
  int ns_b;     // 256-row tiles of the other pairs
  int stage_a;  // pairs with nb 512-row tiles; < 0: no staged layout
  int64_t n_big, n_small;
};

// 256-row tiles that cover the rows of a pair past its first nb 512-row tiles.
constexpr int small_tiles_after(int64_t Nq, int nb) {
  const int64_t left = Nq - int64_t(nb) * 512;
  return left > 0 ? int((left + 255) / 256) : 0;
}

constexpr StagedLayout staged_layout(int64_t Nq, int64_t pairs, int nb, int64_t stage_a) {
  StagedLayout s{};
  s.nb = nb;
  s.ns_a = small_tiles_after(Nq, nb);
  s.ns_b = small_tiles_after(Nq, nb - 1);
  s.stage_a = int(stage_a);
  s.n_big = int64_t(nb - 1) * pairs + stage_a;
  s.n_small = stage_a * s.ns_a + (pairs - stage_a) * s.ns_b;
  return s;
}

// Launches of more 512-row tiles than this many rounds are not searched (a
// staged layout would gain them at most one round in as many).
constexpr int kStagedMaxRounds = 64;

// The staged layout with the earliest estimated finish for `pairs` pairs of Nq
// rows on `cus` compute units (*t_est: its estimate; stage_a < 0 and *t_est =
// 1e300 when there is none to search).  For every nb, the candidates are the
// ends of the range of stage_a and the values that make the 512-row tiles
// fill whole rounds (give or take one).
constexpr StagedLayout plan_staged(int64_t Nq, int64_t pairs, int cus, double c1, double* t_est) {
  StagedLayout best{};
  best.stage_a = -1;
  double t_best = 1e300;
  const int all_big = Nq > 0 ? int((Nq + 511) / 512) : 0;
  if (Nq < 1 || pairs < 1 || cus < 1 || int64_t(all_big) * pairs > int64_t(kStagedMaxRounds) * cus) {
    *t_est = t_best;
    return best;
  }
  for (int nb = 1; nb <= all_big; ++nb) {
    const int64_t base = int64_t(nb - 1) * pairs;  // 512-row tiles at stage_a = 0
    auto consider = [&](int64_t a) {
      if (a < 0 || a > pairs) return;
      const StagedLayout s = staged_layout(Nq, pairs, nb, a);
      const double t = estimated_makespan(s.n_big, s.n_small, cus, c1);
      if (t < t_best - 1e-9) {
        t_best = t;
        best = s;
      }
    };
    consider(0);
    consider(pairs);
    for (int64_t k = base / cus; k <= (base + pairs) / cus + 1; ++k)
      for (int64_t d = -1; d <= 1; ++d) consider(k * cus - base + d);
  }
  *t_est = t_best;
  return best;
}

// Tile `lin` of the 512-row (big) or 256-row tiles of a staged layout, in
// dispatch order within its kind: its pair and first row.
struct StagedTile {
  int64_t pair;
  int64_t row0;
};
constexpr StagedTile staged_tile(int64_t lin, bool big, int nb, int ns_a, int ns_b,
                                 int64_t stage_a) {
  const int64_t per_a = big ? nb : ns_a;
  const int64_t per_b = big ? nb - 1 : ns_b;
  const int64_t in_a = stage_a * per_a;
  int64_t pair = 0, j = 0;
  if (lin < in_a) {
    pair = lin / per_a;
    j = lin % per_a;
  } else {
    const int64_t l2 = lin - in_a, pb = per_b > 0 ? per_b : 1;
    pair = stage_a + l2 / pb;
    j = l2 % pb;
  }
  const int64_t nb_pair = pair < stage_a ? nb : nb - 1;
  return StagedTile{pair, big ? j * 512 : nb_pair * 512 + j * 256};
}

}  // namespace dita
