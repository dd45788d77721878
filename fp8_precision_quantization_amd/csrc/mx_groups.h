// Group tables of the grouped blocked layouts, rebuilt on the device from
// the caller's cumulative END offsets so that no offset is read on the host
// ("[mxfp8 moe training] add compile support", change list).  Shared by the
// layout kernels and the cast that writes M-grouped scales itself.
#pragma once

#include "mx_device.h"
#include "mxcast.h"

namespace mx {

struct GroupTable {
  int32_t lo[MX_MAX_GROUPS];
  int32_t hi[MX_MAX_GROUPS];
  int32_t start[MX_MAX_GROUPS + 1];
};
struct NoTable {};

__device__ __forceinline__ int32_t wave_incl_max(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int32_t o = __shfl_up(v, d);
    if (lane >= d)
      v = max(v, o);
  }
  return v;
}

__device__ __forceinline__ int32_t wave_incl_sum(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int32_t o = __shfl_up(v, d);
    if (lane >= d)
      v += o;
  }
  return v;
}

// Wave 0 fills the table: end_g = min(max(0, ends_0 .. ends_g), extent),
// lo_g = end_{g-1} (lo_0 = 0), start_g = sum over h < g of
// round_up(end_h - lo_h, unit), start_G = padded total.  Lane l handles the
// groups [l * per, (l + 1) * per).
__device__ inline void build_group_table(const int32_t* __restrict__ ends, int groups, int32_t extent,
                                  int32_t unit, GroupTable& t) {
  const int lane = threadIdx.x & 63;
  const int per = (groups + 63) / 64;
  const int g0 = min(lane * per, groups), g1 = min(g0 + per, groups);
  int32_t run = 0;
  for (int g = g0; g < g1; ++g) {
    run = max(run, ends[g]);
    t.hi[g] = run;
  }
  int32_t incl = wave_incl_max(run, lane);
  int32_t excl = __shfl_up(incl, 1);
  if (lane == 0)
    excl = 0;
  int32_t prev = min(excl, extent);
  int32_t local = 0;
  for (int g = g0; g < g1; ++g) {
    int32_t e = min(max(excl, t.hi[g]), extent);
    t.lo[g] = prev;
    t.hi[g] = e;
    local += (e - prev + unit - 1) / unit * unit;
    prev = e;
  }
  int32_t sincl = wave_incl_sum(local, lane);
  int32_t sexcl = sincl - local;
  for (int g = g0; g < g1; ++g) {
    t.start[g] = sexcl;
    sexcl += (t.hi[g] - t.lo[g] + unit - 1) / unit * unit;
  }
  int32_t total = __shfl(sincl, 63);
  if (lane == 0)
    t.start[groups] = total;
}

// The same table for a few groups, by one wave in a uniform loop: the ends
// are read with scalar loads, which every workgroup after the first on a CU
// finds in the scalar cache (the vector loads of build_group_table go to the
// L2 each time, a round trip the grouped layouts wait for before their
// first data load).  Lane 0 writes the table.
constexpr int kScalarTableGroups = 32;
__device__ inline void build_group_table_scalar(const int32_t* __restrict__ ends, int groups, int32_t extent,
                                                int32_t unit, GroupTable& t) {
  const bool writer = (threadIdx.x & 63) == 0;
  int32_t run = 0, prev = 0, start = 0;
  for (int g = 0; g < groups; ++g) {
    run = max(run, ends[g]);
    const int32_t e = min(run, extent);
    if (writer) {
      t.lo[g] = prev;
      t.hi[g] = e;
      t.start[g] = start;
    }
    start += (e - prev + unit - 1) / unit * unit;
    prev = e;
  }
  if (writer)
    t.start[groups] = start;
}

// Last g in [0, groups) with start[g] <= pos, or -1 if pos >= start[groups].
__device__ __forceinline__ int find_group(const GroupTable& t, int groups, int32_t pos) {
  if (pos >= t.start[groups])
    return -1;
  int lo = 0, hi = groups;  // invariant: start[lo] <= pos < start[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (t.start[mid] <= pos)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Group holding row (or column) pos of the source: the g with lo[g] <= pos <
// hi[g], or -1 when pos is at or past the last clamped end.
__device__ __forceinline__ int find_source_group(const GroupTable& t, int groups, int32_t pos) {
  if (groups <= 0 || pos >= t.hi[groups - 1])
    return -1;
  int lo = 0, hi = groups - 1;  // smallest g with hi[g] > pos lies in [lo, hi]
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (t.hi[mid] > pos)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// Starts of each group's piece of an XCD's work in the grouped GEMM: group g
// has T_g = (start[g + 1] - start[g]) / unit * tiles_n tiles, cut into 8
// pieces of P_g = ceil(T_g / 8) (one per XCD); xs[g] = sum of the earlier
// P_h, xs[G] the total.  Wave 0 fills it after the row table.
__device__ inline void build_piece_starts(const GroupTable& t, int groups, int32_t unit, uint32_t tiles_n,
                                          int32_t* xs) {
  const int lane = threadIdx.x & 63;
  const int per = (groups + 63) / 64;
  const int g0 = min(lane * per, groups), g1 = min(g0 + per, groups);
  auto pieces = [&](int g) {
    return (int32_t)(((uint32_t)((t.start[g + 1] - t.start[g]) / unit) * tiles_n + 7) / 8);
  };
  int32_t local = 0;
  for (int g = g0; g < g1; ++g)
    local += pieces(g);
  const int32_t incl = wave_incl_sum(local, lane);
  int32_t run = incl - local;
  for (int g = g0; g < g1; ++g) {
    xs[g] = run;
    run += pieces(g);
  }
  const int32_t total = __shfl(incl, 63);
  if (lane == 0)
    xs[groups] = total;
}

// Starts of the K-grouped blocked scales of row groups: group g covers scale
// columns (32-row blocks) [lo_g / 32, hi_g / 32) of its clamped row range,
// padded to a multiple of 4; kstart[g] = sum of the earlier padded widths,
// kstart[G] the total.  Wave 0 fills it after the row table (the cast that
// writes K-grouped column scales, and the GEMM grouped along K that reads
// them).
struct KStarts {
  int32_t start[MX_MAX_GROUPS + 1];
};
struct NoKStarts {};

__device__ inline void build_kstarts(const GroupTable& t, int groups, KStarts& k) {
  const int lane = threadIdx.x & 63;
  const int per = (groups + 63) / 64;
  const int g0 = min(lane * per, groups), g1 = min(g0 + per, groups);
  int32_t local = 0;
  for (int g = g0; g < g1; ++g)
    local += (t.hi[g] / 32 - t.lo[g] / 32 + 3) / 4 * 4;
  const int32_t incl = wave_incl_sum(local, lane);
  int32_t run = incl - local;
  for (int g = g0; g < g1; ++g) {
    k.start[g] = run;
    run += (t.hi[g] / 32 - t.lo[g] / 32 + 3) / 4 * 4;
  }
  const int32_t total = __shfl(incl, 63);
  if (lane == 0)
    k.start[groups] = total;
}

}  // namespace mx
