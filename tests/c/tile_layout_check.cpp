// Host check of the staged query-tile layout (partial_state_reuse_amd/csrc/
// tile_layout.h) over many launch shapes: for the layout the planner returns,
// every 512-row and 256-row tile is decoded the way the attention kernel
// decodes it (each kind in its own dispatch order), and the tiles must cover
// every query row of every (head, block) pair exactly once, start below Nq,
// and come in the counts the layout states; the planner's estimate must equal
// the makespan model at the layout's tile counts and be no worse than the
// 512-row-only layout (one of its candidates).
#include "../../partial_state_reuse_amd/csrc/tile_layout.h"

#include <cstdio>
#include <vector>

using namespace dita;

static int fail(const char* what, int64_t Nq, int64_t pairs, int cus) {
  std::printf("FAIL %s (Nq=%lld pairs=%lld cus=%d)\n", what, (long long)Nq, (long long)pairs, cus);
  return 1;
}

int main() {
  long shapes = 0, staged = 0;
  for (int cus : {1, 7, 64, 80, 256, 304})
    for (int64_t Nq : {1, 31, 32, 117, 128, 255, 256, 257, 511, 512, 513, 700, 1024, 2048, 2100,
                       4001, 4095, 4725, 5120, 9000})
      for (int64_t pairs : {1, 2, 3, 12, 40, 41, 80, 120, 240, 640, 1000}) {
        ++shapes;
        double t = 0.0;
        const StagedLayout s = plan_staged(Nq, pairs, cus, kSmallTileCost, &t);
        const int all_big = int((Nq + 511) / 512);
        if (int64_t(all_big) * pairs > int64_t(kStagedMaxRounds) * cus) {
          if (s.stage_a >= 0 || t != 1e300) return fail("searched past the round limit", Nq, pairs, cus);
          continue;
        }
        if (s.stage_a < 0 || s.stage_a > pairs) return fail("stage_a range", Nq, pairs, cus);
        if (s.nb < 1 || s.nb > all_big) return fail("nb range", Nq, pairs, cus);
        if (s.n_big != int64_t(s.nb - 1) * pairs + s.stage_a ||
            s.n_small != s.stage_a * s.ns_a + (pairs - s.stage_a) * s.ns_b)
          return fail("tile counts", Nq, pairs, cus);
        if (t != estimated_makespan(s.n_big, s.n_small, cus, kSmallTileCost))
          return fail("estimate", Nq, pairs, cus);
        if (t > estimated_makespan(int64_t(all_big) * pairs, 0, cus, kSmallTileCost) + 1e-9)
          return fail("worse than 512-row tiles only", Nq, pairs, cus);
        if (s.n_small > 0) ++staged;
        // Rows covered per pair, as counts per 32-row block.
        const int64_t blocks = (Nq + 31) / 32;
        std::vector<int> cover(size_t(pairs * blocks), 0);
        for (int kind = 0; kind < 2; ++kind) {
          const bool big = kind == 0;
          const int64_t n = big ? s.n_big : s.n_small;
          for (int64_t lin = 0; lin < n; ++lin) {
            const StagedTile st = staged_tile(lin, big, s.nb, s.ns_a, s.ns_b, s.stage_a);
            if (st.pair < 0 || st.pair >= pairs) return fail("pair range", Nq, pairs, cus);
            if (st.row0 < 0 || st.row0 >= Nq) return fail("tile start", Nq, pairs, cus);
            const int64_t rows = big ? 512 : 256;
            for (int64_t b = st.row0 / 32; b < (st.row0 + rows) / 32 && b < blocks; ++b)
              ++cover[size_t(st.pair * blocks + b)];
          }
        }
        for (int c : cover)
          if (c != 1) return fail("row coverage", Nq, pairs, cus);
      }
  std::printf("ok %ld shapes, %ld with 256-row tiles\n", shapes, staged);
  return 0;
}
