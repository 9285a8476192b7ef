// Host check of the grouped-GEMM tile schedule (csrc/tile_sched.h): for many
// shapes, the units of all workgroups cover every (row tile, weight tile)
// exactly once and, per tile, partition its K units into disjoint ranges;
// no XCD has more units than the grid provides; tail splits stay within
// split_max and the concurrent slots.  Prints "ok <cases>" or the first
// failure, and exits non-zero on failure.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "tile_sched.h"

using namespace moe;

static int check(int Mreal, int nt, int gm, int gn, int kunits, int slots, int split_max) {
  const int64_t R = (int64_t)Mreal * nt;
  std::vector<int> cover((size_t)R * kunits, 0);
  const int64_t per_xcd = sched_units_bound(R, slots);
  for (int x = 0; x < kNumXcd; ++x) {
    int64_t units = 0;
    for (int64_t i = 0; i < per_xcd + 3; ++i) {
      SchedUnit u{};
      const bool ok = sched_unit(Mreal, nt, gm, gn, kunits, slots, split_max, x, i, u);
      if (!ok) continue;
      if (i >= per_xcd) {
        printf("FAIL unit beyond grid M=%d nt=%d x=%d i=%lld\n", Mreal, nt, x, (long long)i);
        return 1;
      }
      ++units;
      if (u.mslot < 0 || u.mslot >= Mreal || u.ntile < 0 || u.ntile >= nt || u.nk <= 0 ||
          u.kbeg < 0 || u.kbeg + u.nk > kunits) {
        printf("FAIL bad unit M=%d nt=%d x=%d i=%lld -> %d %d %d %d\n", Mreal, nt, x,
               (long long)i, u.mslot, u.ntile, u.kbeg, u.nk);
        return 1;
      }
      if (u.nk < kunits / split_max) {
        printf("FAIL split beyond split_max M=%d nt=%d\n", Mreal, nt);
        return 1;
      }
      for (int k = u.kbeg; k < u.kbeg + u.nk; ++k)
        cover[((size_t)u.mslot * nt + u.ntile) * kunits + k]++;
    }
    if (units != sched_units_of_xcd(R, x, slots, split_max)) {
      printf("FAIL unit count M=%d nt=%d x=%d\n", Mreal, nt, x);
      return 1;
    }
  }
  for (size_t c = 0; c < cover.size(); ++c)
    if (cover[c] != 1) {
      printf("FAIL cover M=%d nt=%d kunits=%d slots=%d split=%d at %zu: %d\n", Mreal, nt,
             kunits, slots, split_max, c, cover[c]);
      return 1;
    }
  return 0;
}

int main() {
  int cases = 0;
  const int Ms[] = {1, 2, 3, 7, 8, 9, 15, 16, 17, 33, 35, 40, 67, 131, 256, 370};
  const int nts[] = {1, 2, 3, 4, 5, 7, 8, 16, 17, 56, 112};
  const int kus[] = {1, 4, 7, 64, 224};
  const int slotss[] = {1, 3, 32, 64};
  const int splits[] = {1, 2, 56};
  for (int M : Ms)
    for (int nt : nts)
      for (int ku : kus)
        for (int sl : slotss)
          for (int sp : splits)
            for (int g = 0; g < 3; ++g) {
              const int gm = g == 0 ? 8 : g == 1 ? 4 : 1, gn = g == 0 ? 4 : g == 1 ? 8 : 16;
              if (check(M, nt, gm, gn, ku, sl, sp < ku ? sp : ku)) return 1;
              ++cases;
            }
  // the blocked order: consecutive tiles of a full block share row tiles
  // within groups of 8 and weight tiles within groups of 4
  for (int64_t q = 0; q < 32; ++q) {
    int m = 0, n = 0;
    sched_tile_of(q, 40, 112, 8, 4, m, n);
    if (m != (int)(q % 8) || n != (int)(q / 8)) {
      printf("FAIL block order q=%lld -> %d %d\n", (long long)q, m, n);
      return 1;
    }
  }
  printf("ok %d\n", cases);
  return 0;
}
