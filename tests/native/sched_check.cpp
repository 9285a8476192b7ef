// Host check of the grouped-GEMM tile schedule (csrc/tile_sched.h): for many
// shapes and per-segment row-tile counts (empty segments included), the units
// of all workgroups cover every (row tile, weight tile) exactly once and, per
// tile, partition its K units into disjoint ranges; every row tile maps to
// the segment that owns it; no XCD has more units than the grid provides;
// tail pieces are no shorter than split_max allows.  Prints "ok <cases>" or
// the first failure, and exits non-zero on failure.
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "tile_sched.h"

using namespace moe;

static int check(const std::vector<int>& tiles_per_seg, int nt, int gn, int kunits, int slots,
                 int split_max, bool nfast) {
  const int nseg = (int)tiles_per_seg.size();
  std::vector<int> pre(nseg + 1, 0);
  for (int s = 0; s < nseg; ++s) pre[s + 1] = pre[s] + tiles_per_seg[s];
  const int Mreal = pre[nseg];
  const int64_t R = (int64_t)Mreal * nt;
  std::vector<int> cover((size_t)R * kunits, 0);
  std::vector<int> tile_seen((size_t)R, 0);
  const int64_t per_xcd = sched_units_bound(R, slots);
  for (int x = 0; x < kNumXcd; ++x) {
    int64_t units = 0;
    for (int64_t i = 0; i < per_xcd + 3; ++i) {
      SchedUnit u{};
      if (!sched_unit(R, kunits, slots, split_max, x, i, u)) continue;
      if (i >= per_xcd) {
        printf("FAIL unit beyond grid M=%d nt=%d x=%d i=%lld\n", Mreal, nt, x, (long long)i);
        return 1;
      }
      ++units;
      int seg = -1, m = -1, n = -1;
      sched_tile_of(u.q, pre.data(), nseg, nt, gn, seg, m, n, nfast);
      if (u.q < 0 || u.q >= R || seg < 0 || seg >= nseg || m < pre[seg] || m >= pre[seg + 1] ||
          n < 0 || n >= nt || u.nk <= 0 || u.kbeg < 0 || u.kbeg + u.nk > kunits) {
        printf("FAIL bad unit M=%d nt=%d gn=%d x=%d i=%lld -> q=%lld seg=%d m=%d n=%d k=%d+%d\n",
               Mreal, nt, gn, x, (long long)i, (long long)u.q, seg, m, n, u.kbeg, u.nk);
        return 1;
      }
      {  // tail bookkeeping: the unit's tail index names its tile and piece
        int64_t qtail = 0;
        int rem = 0, S = 0;
        sched_tail_of_xcd(R, x, slots, split_max, qtail, rem, S);
        if (u.S != (u.tail >= 0 ? S : u.S) || (u.tail >= 0) != (u.q >= qtail && S > 1) ||
            (u.tail >= 0 && (u.tail >= rem * S || qtail + u.tail / S != u.q ||
                             u.tail >= slots))) {
          printf("FAIL tail bookkeeping M=%d nt=%d x=%d i=%lld\n", Mreal, nt, x, (long long)i);
          return 1;
        }
      }
      if (u.nk < kunits / split_max) {
        printf("FAIL piece shorter than split_max allows M=%d nt=%d\n", Mreal, nt);
        return 1;
      }
      for (int k = u.kbeg; k < u.kbeg + u.nk; ++k) cover[((size_t)m * nt + n) * kunits + k]++;
    }
    if (units != sched_units_of_xcd(R, x, slots, split_max)) {
      printf("FAIL unit count M=%d nt=%d x=%d\n", Mreal, nt, x);
      return 1;
    }
  }
  for (size_t c = 0; c < cover.size(); ++c)
    if (cover[c] != 1) {
      printf("FAIL cover M=%d nt=%d gn=%d kunits=%d slots=%d split=%d at %zu: %d\n", Mreal, nt,
             gn, kunits, slots, split_max, c, cover[c]);
      return 1;
    }
  // the tile map alone is a bijection q <-> (row tile, weight tile)
  for (int64_t q = 0; q < R; ++q) {
    int seg = -1, m = -1, n = -1;
    sched_tile_of(q, pre.data(), nseg, nt, gn, seg, m, n, nfast);
    tile_seen[(size_t)m * nt + n]++;
  }
  for (size_t c = 0; c < tile_seen.size(); ++c)
    if (tile_seen[c] != 1) {
      printf("FAIL tile map not a bijection M=%d nt=%d gn=%d\n", Mreal, nt, gn);
      return 1;
    }
  return 0;
}

int main() {
  int cases = 0;
  std::mt19937 rng(12345);
  const int nsegs[] = {1, 2, 3, 8, 9, 65, 257};
  const int nts[] = {1, 3, 4, 7, 8, 16, 17, 56};
  const int kus[] = {1, 7, 64, 224};
  const int slotss[] = {1, 3, 32};
  const int splits[] = {1, 2, 56};
  const int gns[] = {1, 4, 8, 16};
  for (int nseg : nsegs)
    for (int shape = 0; shape < 3; ++shape) {
      // row tiles per segment: uniform small, skewed with empty segments, all 1
      std::vector<int> tps(nseg);
      for (int s = 0; s < nseg; ++s) {
        if (shape == 0) tps[s] = 1 + (int)(rng() % 5);
        else if (shape == 1) tps[s] = (rng() % 3 == 0) ? 0 : (int)(rng() % 4);
        else tps[s] = 1;
      }
      if (shape == 1) tps[0] = 3;  // at least one tile
      for (int nt : nts)
        for (int gn : gns)
          for (int ku : kus)
            for (int sl : slotss)
              for (int sp : splits) {
                if (nseg * nt > 4000 && (ku > 7 || sl != 32)) continue;  // keep it quick
                for (int nf = 0; nf < 2; ++nf) {
                  if (check(tps, nt, gn, ku, sl, sp < ku ? sp : ku, nf != 0)) return 1;
                  ++cases;
                }
              }
    }
  // expert-aligned blocks: with segments of 4 row tiles and gn = 8, the first
  // 32 tiles are segment 0's 4 row tiles x weight tiles 0..7
  std::vector<int> pre = {0, 4, 8, 12};
  for (int64_t q = 0; q < 32; ++q) {
    int seg = -1, m = -1, n = -1;
    sched_tile_of(q, pre.data(), 3, 112, 8, seg, m, n);
    if (seg != 0 || m != (int)(q % 4) || n != (int)(q / 4)) {
      printf("FAIL block order q=%lld -> seg %d m %d n %d\n", (long long)q, seg, m, n);
      return 1;
    }
  }
  // weight tiles fastest: the first 32 tiles are row tiles 0..3 of segment 0,
  // each with weight tiles 0..7
  for (int64_t q = 0; q < 32; ++q) {
    int seg = -1, m = -1, n = -1;
    sched_tile_of(q, pre.data(), 3, 112, 8, seg, m, n, true);
    if (seg != 0 || m != (int)(q / 8) || n != (int)(q % 8)) {
      printf("FAIL nfast block order q=%lld -> seg %d m %d n %d\n", (long long)q, seg, m, n);
      return 1;
    }
  }
  printf("ok %d\n", cases);
  return 0;
}
