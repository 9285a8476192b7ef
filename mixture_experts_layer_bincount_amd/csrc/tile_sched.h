// Work schedule of the grouped expert GEMMs: which output tile (and which
// range of K) a workgroup computes.
//
// The number of row tiles is only known on the device (it depends on the
// per-expert counts that the dispatch wrote), so every workgroup derives its
// unit from the device-side total:
//
//  * Real tiles are numbered densely, q = 0 .. R-1 with R = Mreal * nt
//    (Mreal row tiles summed over the expert segments, nt weight tiles), in
//    expert-aligned blocks: the weight tiles are taken in groups of gn, and
//    inside a group segment by segment, all row tiles of the segment times
//    the group's weight tiles, either row tiles fastest (consecutive q share
//    a weight panel) or weight tiles fastest (nfast: the gn consecutive q of
//    one row tile share its activation rows, and do the same work, so they
//    run in step).  A block never mixes two experts' weights.
//  * Workgroup ids are dealt round-robin to the XCDs; XCD x takes the
//    contiguous q range [R x / X, R (x+1) / X), so every XCD gets the same
//    number of tiles (+-1) and its concurrent workgroups stay inside one or
//    two operand blocks.
//  * An XCD runs `slots` workgroups at once.  Its tiles fill
//    floor(n / slots) whole rounds; when splitting is allowed (partial sums
//    that are added, as the atomic combine does) the tiles of the last,
//    partial round are cut into S K-ranges with rem * S <= slots, so the tail
//    round takes 1/S of a tile's time instead of a whole one.
//
// Everything here is constexpr (callable from host and device code) and
// free of HIP types, so the arithmetic is checked by a host-compiled test.
#pragma once

#include <stdint.h>

namespace moe {

constexpr int kNumXcd = 8;  // XCDs of an MI355X; workgroups are dealt round-robin

struct SchedUnit {
  int64_t q;  // tile, 0 .. R-1
  int kbeg;   // first K unit
  int nk;     // K units
  int S;      // K pieces of the tile (1: a whole tile)
  int tail;   // for a piece of a split tile: its index among the XCD's tail
              // units, rem * S <= slots of them (-1 for a whole tile)
};

// Tile q -> (segment, row tile, weight tile) in the expert-aligned order
// described above.  pre[s] is the first row tile of segment s (exclusive
// prefix sum of the segments' row tiles, pre[nseg] = Mreal); empty segments
// are allowed.
constexpr void sched_tile_of(int64_t q, const int* pre, int nseg, int nt, int gn, int& seg,
                             int& mslot, int& ntile, bool nfast = false) {
  const int Mreal = pre[nseg];
  const int64_t col = (int64_t)Mreal * gn;  // tiles per full weight-tile group
  const int ng = (int)(q / col);
  const int64_t r = q - (int64_t)ng * col;
  const int nh = (nt - ng * gn) < gn ? (nt - ng * gn) : gn;
  // the last segment s with pre[s] * nh <= r (it is never empty)
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)pre[mid] * nh <= r) lo = mid; else hi = mid - 1;
  }
  seg = lo;
  const int me = pre[seg + 1] - pre[seg];
  const int64_t loc = r - (int64_t)pre[seg] * nh;
  if (nfast) {
    mslot = pre[seg] + (int)(loc / nh);
    ntile = ng * gn + (int)(loc % nh);
  } else {
    mslot = pre[seg] + (int)(loc % me);
    ntile = ng * gn + (int)(loc / me);
  }
}

// The K-range split of the tail round: pieces per tile for `rem` tiles on
// `slots` concurrent workgroups, at most `split_max`.
constexpr int sched_tail_split(int rem, int slots, int split_max) {
  if (rem <= 0) return 1;
  int s = slots / rem;
  if (s > split_max) s = split_max;
  return s < 1 ? 1 : s;
}

// Units one XCD runs (tiles of its whole rounds plus split tail pieces).
constexpr int64_t sched_units_of_xcd(int64_t R, int xcd, int slots, int split_max) {
  const int64_t q0 = R * xcd / kNumXcd, q1 = R * (xcd + 1) / kNumXcd;
  const int64_t n = q1 - q0;
  const int64_t full = n / slots * slots;
  const int rem = (int)(n - full);
  return full + (int64_t)rem * sched_tail_split(rem, slots, split_max);
}

// The XCD's tail: its tiles after the whole rounds (rem), and the K pieces
// each is cut into (S); tail unit j = r * S + piece covers tile q0 + full + r.
constexpr void sched_tail_of_xcd(int64_t R, int xcd, int slots, int split_max, int64_t& qtail,
                                 int& rem, int& S) {
  const int64_t q0 = R * xcd / kNumXcd, q1 = R * (xcd + 1) / kNumXcd;
  const int64_t n = q1 - q0;
  const int64_t full = n / slots * slots;
  qtail = q0 + full;
  rem = (int)(n - full);
  S = sched_tail_split(rem, slots, split_max);
}

// Upper bound of the units of any XCD given an upper bound of R (grid size).
constexpr int64_t sched_units_bound(int64_t R_max, int slots) {
  return (R_max + kNumXcd - 1) / kNumXcd + slots;
}

// Unit of workgroup `i` of XCD `xcd` among R tiles.  kunits: K units of a
// whole tile.  Returns false when the workgroup has nothing to do.
constexpr bool sched_unit(int64_t R, int kunits, int slots, int split_max, int xcd, int64_t i,
                          SchedUnit& u) {
  const int64_t q0 = R * xcd / kNumXcd, q1 = R * (xcd + 1) / kNumXcd;
  const int64_t n = q1 - q0;
  const int64_t full = n / slots * slots;
  int piece = 0, S = 1;
  u.tail = -1;
  if (i < full) {
    u.q = q0 + i;
  } else {
    const int rem = (int)(n - full);
    S = sched_tail_split(rem, slots, split_max);
    const int64_t j = i - full;
    if (j >= (int64_t)rem * S) return false;
    u.q = q0 + full + j / S;
    piece = (int)(j % S);
    if (S > 1) u.tail = (int)j;
  }
  u.S = S;
  u.kbeg = (int)((int64_t)kunits * piece / S);
  u.nk = (int)((int64_t)kunits * (piece + 1) / S) - u.kbeg;
  return true;
}

}  // namespace moe
