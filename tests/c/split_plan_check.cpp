// Host check of the key-split planner (partial_state_reuse_amd/csrc/split_plan.h)
// over many launch shapes: every plan the planner returns is decoded the way the
// attention kernel decodes it (each unit's first segment to the end of the tile
// it starts in, then the start of the next tile), and the decode must cover
// every (tile, key-tile) iteration exactly once, keep every segment inside one
// tile, give every piece a distinct scratch slot below 2U, index counters below
// rem, and produce exactly split_pieces(r) pieces of each tile (none for a tile
// that one unit covers whole), at most kSplitMaxPieces.
#include "../../partial_state_reuse_amd/csrc/split_plan.h"

#include <cstdio>
#include <set>
#include <vector>

using namespace dita;

static int fail(const char* what, int64_t n, int cus, int T) {
  std::printf("FAIL %s (n=%lld cus=%d T=%d)\n", what, (long long)n, cus, T);
  return 1;
}

int main() {
  long planned = 0, shapes = 0;
  for (int cus : {1, 7, 64, 80, 256, 304})
    for (int64_t n = 1; n <= 3000; n += (n < 300 ? 1 : 37))
      for (int T : {1, 2, 3, 5, 9, 74, 148, 150, 1000}) {
        ++shapes;
        double t = -1.0;
        const SplitPlan p = plan_key_split(n, cus, T, 4, &t);
        if (p.units == 0) continue;
        ++planned;
        if (p.rem != n % cus || p.G != int64_t(p.rem) * T || p.units <= p.rem ||
            p.units > cus || p.units > kSplitMaxUnits || p.rem > kSplitMaxCounters)
          return fail("plan fields", n, cus, T);
        if (!(t >= double(n / cus)) || !(t <= double(n / cus) + 1.0 + 8.0 / T + 1e-9))
          return fail("estimate", n, cus, T);
        std::vector<int> cover(size_t(p.G), 0);
        std::vector<int> seen(size_t(p.rem), 0);
        std::set<int64_t> slots;
        for (int64_t u = 0; u < p.units; ++u) {
          const int64_t x = split_lo(p, u), hi = split_lo(p, u + 1);
          if (hi <= x || hi - x > T) return fail("unit length", n, cus, T);
          const int64_t edge = split_edge(p, u);
          const int64_t r = x / T;
          const int64_t k0 = x - r * T, k1 = (hi < edge ? hi : edge) - r * T;
          if (r >= p.rem || k1 <= k0 || k1 > T) return fail("first segment", n, cus, T);
          for (int64_t k = k0; k < k1; ++k) ++cover[size_t(r * T + k)];
          if (!(k0 == 0 && k1 == T)) {
            if (split_slot(p, u, r) != 2 * u || !slots.insert(2 * u).second)
              return fail("first slot", n, cus, T);
            ++seen[size_t(r)];
          }
          if (split_has_second(p, u)) {
            const int64_t r2 = r + 1, k2 = hi - r2 * T;
            if (r2 >= p.rem || k2 <= 0 || k2 >= T) return fail("second segment", n, cus, T);
            for (int64_t k = 0; k < k2; ++k) ++cover[size_t(r2 * T + k)];
            if (split_slot(p, u, r2) != 2 * u + 1 || !slots.insert(2 * u + 1).second)
              return fail("second slot", n, cus, T);
            ++seen[size_t(r2)];
          }
        }
        for (int c : cover)
          if (c != 1) return fail("coverage", n, cus, T);
        for (int64_t r = 0; r < p.rem; ++r) {
          const int np = split_pieces(p, r);
          if (np > kSplitMaxPieces || (np == 1 ? seen[size_t(r)] != 0 : seen[size_t(r)] != np))
            return fail("pieces", n, cus, T);
          if (split_first_unit(p, r) != split_unit_of(p, r * T)) return fail("first unit", n, cus, T);
        }
      }
  std::printf("ok %ld shapes, %ld split\n", shapes, planned);
  return planned > 0 ? 0 : 1;
}
