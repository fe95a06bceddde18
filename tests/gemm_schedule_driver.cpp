// Host test driver for the persistent GEMM's tile schedule: reads launches
// from stdin, one per line ("grid np tiles[0..np) ktiles[0..np)"), and
// prints for each either "none" or, per XCD x, problem p and workgroup l
// with a nonzero count, "x p l count position...", the positions of its
// tiles within XCD x's share of problem p in the order the kernel runs
// them.  Built with g++ by tests/test_gemm_schedule.py.
#include <cstdio>

#include "gemm_schedule.h"

using namespace fp8l::sched;

int main() {
  int grid, np;
  while (std::scanf("%d %d", &grid, &np) == 2) {
    int tiles[MAX_PROBLEMS] = {}, ktiles[MAX_PROBLEMS] = {};
    for (int p = 0; p < 2 * np; ++p) {
      int v = 0;
      if (std::scanf("%d", &v) != 1) return 1;
      if (p < np && p < MAX_PROBLEMS) tiles[p] = v;
      if (p >= np && p - np < MAX_PROBLEMS) ktiles[p - np] = v;
    }
    Packed pk;
    if (!balance(grid, np, tiles, ktiles, pk)) {
      std::printf("none\n");
      continue;
    }
    for (int x = 0; x < XCDS; ++x) {
      const int nx = xcd_workgroups(grid, x);
      for (int p = 0; p < np; ++p)
        for (int l = 0; l < nx; ++l) {
          const int cnt = pk.entry[x][p][l] & 255, extra = pk.entry[x][p][l] >> 8;
          if (cnt == 0) continue;
          std::printf("%d %d %d %d", x, p, l, cnt);
          for (int i = 0; i < cnt; ++i)
            std::printf(" %d", position(i, l, nx, pk.min_count[x][p], extra));
          std::printf("\n");
        }
    }
    std::printf("end\n");
  }
  return 0;
}
