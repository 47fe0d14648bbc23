// Key-split work units for the query tiles of the last, partial round of an
// attention launch.
//
// A launch of n query tiles on C compute units (one tile per unit at a time)
// runs floor(n / C) full rounds and a last round in which only n mod C units
// work.  The tiles of that last round (the "remainder", rem of them) are
// instead spread over U <= C workgroups ("units") along the key axis: the rem
// tiles form one sequence of rem * T key-tile iterations (T per tile), and
// unit u takes the contiguous range [lo(u), lo(u + 1)) with lo(u) =
// floor(u * rem * T / U).  A unit's range crosses tile boundaries, so a tile
// can be computed in pieces by consecutive units; each piece is the exact
// attention state of the tile's queries against a contiguous key range, and
// the LSE merge of the pieces is the tile's state over all its keys (the state
// composition of the DiTango page, State-Centric Parallel Runtime > State
// Composition, applied to sub-ranges of one partition).
//
// Every function is constexpr, so it serves the host planner and the device
// kernel alike.
#pragma once

#include <algorithm>
#include <cstdint>

namespace dita {

// Value-initialise (SplitPlan{}) for "no split": the struct is trivial so that
// it can live in LDS.
struct SplitPlan {
  int units;   // U; 0: no key split in this launch
  int rem;     // remainder tiles shared by the units
  int T;       // key-tile iterations per query tile
  int64_t G;   // rem * T
};

// First iteration of unit u (u = U gives G).
constexpr int64_t split_lo(const SplitPlan& p, int64_t u) { return u * p.G / p.units; }

// Unit whose range holds iteration x (0 <= x < G): the largest u with lo(u) <= x.
constexpr int64_t split_unit_of(const SplitPlan& p, int64_t x) {
  return ((x + 1) * p.units - 1) / p.G;
}

// Units that compute a piece of remainder tile r: [first, first + count).
constexpr int64_t split_first_unit(const SplitPlan& p, int64_t r) {
  return split_unit_of(p, r * p.T);
}
constexpr int split_pieces(const SplitPlan& p, int64_t r) {
  return int(split_unit_of(p, r * p.T + p.T - 1) - split_unit_of(p, r * p.T) + 1);
}

// Scratch slot of unit u's piece of tile r: every unit holds at most two
// pieces, the end of the tile its range starts in (slot 2u) and the start of
// the tile its range ends in (slot 2u + 1); tiles it covers whole are not
// pieces.  A range inside one tile is a single piece in slot 2u.
constexpr int64_t split_slot(const SplitPlan& p, int64_t u, int64_t r) {
  return 2 * u + (split_lo(p, u) / p.T == r ? 0 : 1);
}

// Segments of unit u: its range [x, hi) is at most a tile long (U > rem), so
// it holds the end of the tile it starts in, [x, min(hi, edge)), and, when it
// crosses edge = the next tile boundary, the start of the next, [edge, hi).
// (A range that is exactly one tile is that whole tile, not a piece.)
constexpr int64_t split_edge(const SplitPlan& p, int64_t u) {
  return (split_lo(p, u) / p.T + 1) * p.T;
}
constexpr bool split_has_second(const SplitPlan& p, int64_t u) {
  return split_lo(p, u + 1) > split_edge(p, u);
}

// Host planning limits.
constexpr int kSplitMaxUnits = 256;                 // units per launch
constexpr int kSplitMaxPieces = 8;                  // pieces of one tile
constexpr int kSplitMaxUnitsPerTile = 6;            // a unit covers at least a sixth of a tile
// More than 4 units per tile only where each still gets at least this many key
// tiles: a unit's fixed costs (its Q tile, the pipeline's restart, storing its
// piece and the combination reading one more) outweigh shorter ranges
// (measured: 4725 x 2000 keys, 30 heads, 7 pieces a tile: 9% slower than 4).
constexpr int kSplitMinIters = 40;
constexpr int kSplitMaxCounters = 4096;             // remainder tiles per launch

// Key split of the last round of n tiles with T key-tile iterations each on
// `cus` compute units (one tile at a time each), with `segment_cost`
// iterations of overhead per segment.  Returns the plan (units == 0: no
// split) and its estimated finishing time in tile times (*t_est): the whole
// rounds, then one unit's range in two segments.  More units than remainder
// tiles, so a unit's range is shorter than a tile; 4 units per tile at most,
// up to kSplitMaxUnitsPerTile for long key ranges (kSplitMinIters), and at
// most kSplitMaxPieces pieces per tile.
inline SplitPlan plan_key_split(int64_t n, int cus, int T, int segment_cost, double* t_est) {
  SplitPlan none{};
  if (cus < 1 || T < 2) return none;
  const int64_t rem = n % cus;
  if (rem == 0 || rem > kSplitMaxCounters) return none;
  const int per_tile = std::max(4, std::min(kSplitMaxUnitsPerTile, T / kSplitMinIters));
  const int64_t top = std::min<int64_t>(std::min(cus, kSplitMaxUnits), rem * std::min(per_tile, T));
  for (int64_t U = top; U > rem; --U) {
    SplitPlan c{};
    c.units = int(U);
    c.rem = int(rem);
    c.T = T;
    c.G = rem * T;
    int most = 0;
    for (int64_t r = 0; r < rem; ++r) most = std::max(most, split_pieces(c, r));
    if (most > kSplitMaxPieces) continue;
    const int64_t longest = (c.G + U - 1) / U;
    *t_est = double(n / cus) + double(longest + 2 * segment_cost) / double(T);
    return c;
  }
  return none;
}

}  // namespace dita
