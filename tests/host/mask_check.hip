// Host-side driver for the kernels' visibility helpers (tree_entry_ok,
// tree_branch_mask, tile_visible in mla_common.h), so that their bit logic can
// be checked on a machine without a GPU. Reads commands from stdin, one per
// line, and prints one result line for each:
//   V ts lim t_draft t1 branch   -> tile_visible(...) as an unsigned decimal
//   T Q p0 p1 ... p(Q-1)         -> Q masks tree_branch_mask(p, Q, j), then
//                                   1/0 for every entry's tree_entry_ok
//   N t0 t1 tile tree t_draft jmax -> tiles_needed(...)
#include <cstdio>
#include <cinttypes>
#include <vector>

#include "mla_common.h"

int main() {
  char op[4];
  while (std::scanf("%3s", op) == 1) {
    if (op[0] == 'V') {
      int ts, lim, t_draft, t1;
      unsigned long long branch;
      if (std::scanf("%d %d %d %d %llu", &ts, &lim, &t_draft, &t1, &branch) != 5) return 2;
      std::printf("%llu\n", (unsigned long long)mla::tile_visible(ts, lim, t_draft, t1, branch));
    } else if (op[0] == 'T') {
      int Q;
      if (std::scanf("%d", &Q) != 1 || Q < 1 || Q > 64) return 2;
      std::vector<int32_t> p(Q);
      for (int i = 0; i < Q; ++i)
        if (std::scanf("%d", &p[i]) != 1) return 2;
      for (int j = 0; j < Q; ++j)
        std::printf("%llu ", (unsigned long long)mla::tree_branch_mask(p.data(), Q, j));
      for (int i = 0; i < Q; ++i) std::printf("%d ", mla::tree_entry_ok(p.data(), i) ? 1 : 0);
      std::printf("\n");
    } else if (op[0] == 'N') {
      int t0, t1, tile, tree, t_draft, jmax;
      if (std::scanf("%d %d %d %d %d %d", &t0, &t1, &tile, &tree, &t_draft, &jmax) != 6) return 2;
      std::printf("%d\n", mla::tiles_needed(t0, t1, tile, tree != 0, t_draft, jmax));
    } else {
      return 2;
    }
  }
  return 0;
}
