// Host-side tile schedule for the persistent GEMM (plain C++, no HIP).
//
// The persistent kernel runs one workgroup per compute unit; workgroup b
// sits on XCD b % 8 and is the (b / 8)-th of that XCD's workgroups.  Each
// problem of a grouped launch deals its tiles to the XCDs round-robin, so
// XCD x owns a contiguous share of every problem's tile order, and the XCD's
// workgroups split that share among themselves.  When the problems of one
// launch have different K, their tiles cost different times, and dealing
// them round-robin leaves some workgroups a whole long tile behind the rest
// (12.5 tiles per workgroup with the long ones last, for instance).  This
// schedule balances the work instead: problems are taken longest-K first,
// and each problem's tiles go one at a time to the workgroup with the least
// work so far (lowest index on ties), the classic longest-processing-time
// list schedule.  The cost of a tile is its number of 128-deep k-tiles plus
// a fixed per-tile overhead (the epilogue and the tile switch, about as long
// as 4 k-tiles).  The result is per XCD, per problem, per workgroup: a count
// of tiles.  The kernel takes an XCD's share of a problem in round order as
// far as every workgroup has tiles (round r: the r-th tile of each
// workgroup, in workgroup order), then each workgroup's extra tiles in
// workgroup order, so the tiles an XCD runs at one time stay neighbours in
// the grouped order.  position() is that order; the kernel and the host
// tests share it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FP8L_SCHED_FN __host__ __device__ inline
#else
#define FP8L_SCHED_FN inline
#endif

namespace fp8l {
namespace sched {

constexpr int XCDS = 8;            // XCDs of the chip; workgroup b on XCD b % 8
constexpr int MAX_WG = 32;         // workgroups per XCD (256 compute units / 8)
constexpr int MAX_PROBLEMS = 4;    // problems of one grouped launch
constexpr int TILE_OVERHEAD = 4;   // per-tile cost beyond its k-tiles, in k-tiles

// Tiles of a problem with `tiles` tiles that XCD x receives when they are
// dealt round-robin.
inline int xcd_share(int tiles, int x) { return (tiles - x + XCDS - 1) / XCDS; }

// Workgroups on XCD x when `grid` workgroups are dealt round-robin.
inline int xcd_workgroups(int grid, int x) { return (grid - x + XCDS - 1) / XCDS; }

// One problem's `cnt` tiles of cost `cost` added to `nx` workgroups whose
// work so far is load[0..nx): tile after tile goes to the least-loaded
// workgroup, lowest index on ties.  Equivalently the cnt smallest of the
// values load[l] + j * cost (j >= 0), ordered by (value, l), are taken;
// found here by bisection on the value.  Writes the count per workgroup to
// out[0..nx) and adds the work to load[].
inline void fill(int nx, int64_t *load, int cnt, int64_t cost, int *out) {
  int64_t lo = load[0], hi = load[0];
  for (int l = 1; l < nx; ++l) {
    lo = load[l] < lo ? load[l] : lo;
    hi = load[l] > hi ? load[l] : hi;
  }
  hi += (int64_t)((cnt + nx - 1) / nx) * cost;   // count_le(hi) >= cnt
  auto count_le = [&](int64_t t) {
    int64_t c = 0;
    for (int l = 0; l < nx; ++l)
      if (load[l] <= t) c += (t - load[l]) / cost + 1;
    return c;
  };
  // smallest t with count_le(t) >= cnt
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (count_le(mid) >= cnt) hi = mid;
    else lo = mid + 1;
  }
  const int64_t t = lo;
  int64_t taken = 0;
  for (int l = 0; l < nx; ++l) {
    out[l] = load[l] <= t - 1 ? (int)((t - 1 - load[l]) / cost + 1) : 0;
    taken += out[l];
  }
  // the values equal to t, in workgroup order, until cnt are taken
  for (int l = 0; l < nx && taken < cnt; ++l)
    if (load[l] <= t && (t - load[l]) % cost == 0) {
      ++out[l];
      ++taken;
    }
  for (int l = 0; l < nx; ++l) load[l] += out[l] * cost;
}

// Position, within XCD x's share of one problem, of the i-th tile of
// workgroup l (0 <= i < its count), for an XCD with nx workgroups whose
// smallest count is mn; extra_before = sum over workgroups l' < l of
// (count[l'] - mn).  Rounds 0..mn-1 take positions r * nx + l; the extra
// tiles follow, workgroup after workgroup.
FP8L_SCHED_FN int position(int i, int l, int nx, int mn, int extra_before) {
  return i < mn ? i * nx + l : mn * nx + extra_before + (i - mn);
}

// A balanced schedule as the kernel reads it: entry = count | extra_before
// << 8 per XCD, problem and workgroup (workgroups past the XCD's count hold
// 0), and the smallest count per XCD and problem.
struct Packed {
  uint16_t entry[XCDS][MAX_PROBLEMS][MAX_WG];
  uint8_t min_count[XCDS][MAX_PROBLEMS];
};

// The schedule of a launch with `np` problems (in the order the kernel takes
// them) of tiles[p] tiles and ktiles[p] k-tiles each, on `grid` workgroups,
// packed: the count in out.entry[x][p][l] is the number of tiles of problem
// p that workgroup l of XCD x runs.
// Returns false (out unspecified) when a count or an offset does not fit a
// byte, or the arguments are out of range; the caller then deals the tiles
// round-robin.
inline bool balance(int grid, int np, const int *tiles, const int *ktiles, Packed &out) {
  if (grid < 1 || grid > XCDS * MAX_WG || np < 1 || np > MAX_PROBLEMS) return false;
  out = Packed{};
  for (int x = 0; x < XCDS; ++x) {
    const int nx = xcd_workgroups(grid, x);
    int64_t load[MAX_WG] = {};
    for (int p = 0; p < np; ++p) {
      int cnt_l[MAX_WG] = {};
      const int cnt = xcd_share(tiles[p], x);
      if (cnt > 0 && nx == 0) return false;   // tiles with no workgroup to run them
      if (nx == 0) continue;
      fill(nx, load, cnt, (int64_t)ktiles[p] + TILE_OVERHEAD, cnt_l);
      int mn = cnt_l[0];
      for (int l = 1; l < nx; ++l) mn = cnt_l[l] < mn ? cnt_l[l] : mn;
      if (mn > 255) return false;
      out.min_count[x][p] = (uint8_t)mn;
      int extra = 0;
      for (int l = 0; l < nx; ++l) {
        if (cnt_l[l] > 255 || extra > 255) return false;
        out.entry[x][p][l] = (uint16_t)(cnt_l[l] | extra << 8);
        extra += cnt_l[l] - mn;
      }
    }
  }
  return true;
}

}  // namespace sched
}  // namespace fp8l
