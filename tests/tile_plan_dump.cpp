// Host program for tests/test_tile_plan.py: prints every work item the tile-range plan of the
// grouped GEMMs (mixture_experts_layer_07_amd/csrc/tile_plan.h) hands out, for the launches given
// on stdin, one per line: total KT min_steps max_slots C. Output per launch: a line
// "L total KT C" and one line "q it tile piece k0 k1 slot first S" per item.
#include <cstdio>

#include "tile_plan.h"

int main() {
  int total, KT, min_steps, max_slots, C;
  while (std::scanf("%d %d %d %d %d", &total, &KT, &min_steps, &max_slots, &C) == 5) {
    std::printf("L %d %d %d\n", total, KT, C);
    for (int q = 0; q < moe::kQueues; ++q) {
      const moe::SplitQueue sq =
          moe::split_plan(q, total, KT, min_steps, max_slots, C, moe::kMaxSplitItems, MOE_MAX_K_PIECES);
      // every workgroup of the range draws until the range is drained: draw past the end too
      for (int it = 0; it < sq.items + C; ++it) {
        const moe::WorkItem w = moe::plan_item(sq, it, KT);
        std::printf("%d %d %d %d %d %d %d %d %d\n", q, it, w.tile, w.piece, w.k0, w.k1, w.slot, w.first, w.S);
      }
    }
  }
  return 0;
}
