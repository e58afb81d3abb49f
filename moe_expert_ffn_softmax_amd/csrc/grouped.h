// Work decomposition shared by the grouped expert GEMM kernels.
//
// A launch covers the routed experts (segments 0..E-1, rows in expert-sorted order)
// and optionally the shared expert (segment E, one row per token).  A work item is
// one row tile of one segment times one or more 32-column groups of its output.
//
// Every workgroup first turns the per-expert counts into a prefix of item counts
// over the segments (in LDS); wave w of the launch then takes items w, w + W,
// w + 2W, ... (W waves in the grid, all resident).  Items of one launch stream
// equal amounts of weights, so static striding balances them; a shared atomic
// queue head was measured slower (thousands of waves contending for one word
// cost more than the imbalance it removes).
#pragma once
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kMaxSegments = 1025;  // E <= 1024 routed + 1 shared

// Per-workgroup LDS copy of the launch's segment table: item-count prefixes and each
// segment's row count and first row.  An item's decode then reads LDS only: the counts
// and offsets in global memory can only be read with vector loads here (the kernels
// store to global memory), and the wait for such a load waits for every load in
// flight, a weight stream's included.
struct SegTable {
  int prefix[kMaxSegments + 1];
  int rows[kMaxSegments];
  int row0[kMaxSegments];
};

struct Item {
  int seg;       // segment (expert, or E for the shared expert)
  bool shared;
  int group;     // 32-column group
  int row0;      // first row of the tile in the segment's output rows
  int nrows;     // rows of the tile (1..tile_rows)
};

// Fill t.prefix[0..S] (S = number of segments) with item-count prefixes, and t.rows
// and t.row0 with each segment's rows; returns the total.  An item covers `tile_rows`
// rows and `groups_per_item` 32-column groups.  Needs blockDim.x / 64 + 1 ints of
// `scan_tmp`.  Contains __syncthreads().
__device__ __forceinline__ int build_item_prefix(const GroupedGemm& g, int tile_rows, int groups_per_item,
                                                 SegTable& t, int* scan_tmp) {
  const int S = g.E + (g.shared_rows > 0 ? 1 : 0);
  int carry = 0;
  for (int s0 = 0; s0 < S; s0 += blockDim.x) {
    const int s = s0 + threadIdx.x;
    int items = 0;
    if (s < S) {
      const bool sh = s >= g.E;
      const int rows = sh ? g.shared_rows : g.counts[s];
      const int groups = sh ? g.groups_shared : g.groups_routed;
      items = (rows + tile_rows - 1) / tile_rows * ((groups + groups_per_item - 1) / groups_per_item);
      t.rows[s] = rows;
      t.row0[s] = sh ? 0 : g.offsets[s];
    }
    int tot = 0;
    const int ex = block_exclusive_scan(items, scan_tmp, &tot);
    if (s < S) t.prefix[s] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) t.prefix[S] = carry;
  __syncthreads();
  return carry;
}

__device__ __forceinline__ int build_item_prefix(const GroupedGemm& g, int tile_rows, SegTable& t, int* scan_tmp) {
  return build_item_prefix(g, tile_rows, 1, t, scan_tmp);
}

__device__ __forceinline__ int find_segment(const GroupedGemm& g, const SegTable& t, int item) {
  const int* prefix = t.prefix;
  const int S = g.E + (g.shared_rows > 0 ? 1 : 0);
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= item)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Item order: segment, row tile, column group fastest (one group per item).  `item` must
// be the same for every lane of the wave.
__device__ __forceinline__ Item decode_item(const GroupedGemm& g, int tile_rows, const SegTable& t, int item) {
  Item it;
  it.seg = __builtin_amdgcn_readfirstlane(find_segment(g, t, item));  // uniform over the wave, as item is
  it.shared = it.seg >= g.E;
  const int local = item - t.prefix[it.seg];
  const int groups = it.shared ? g.groups_shared : g.groups_routed;
  const int tile = local / groups;
  it.group = local - tile * groups;
  const int rows = t.rows[it.seg];
  it.row0 = t.row0[it.seg] + tile * tile_rows;
  it.nrows = min(tile_rows, rows - tile * tile_rows);
  return it;
}

// Item order: segment, column tile, row tile fastest, so the row tiles of one expert
// that read the same weights are neighbours and run at the same time.  A segment's
// rows are split evenly over its row tiles (155 rows: 78 + 77, not 128 + 27): tiles
// of equal fill run at equal speed, so the partner tiles of a column tile stay close
// enough for the second one's weight loads to hit the first one's lines in L2.  (With
// a full tile beside a nearly empty one the faster tile ran ahead and the pair fetched
// the expert's weights twice: on MI355X, layers with ~100-150 rows per expert fetched
// 34-45% more than their weight bytes into L2; with even splits 13-15%.)  `group` is
// the first group of the item.
__device__ __forceinline__ Item decode_item_tiled(const GroupedGemm& g, int tile_rows, int groups_per_item,
                                                  const SegTable& t, int item) {
  Item it;
  it.seg = __builtin_amdgcn_readfirstlane(find_segment(g, t, item));  // as in decode_item
  it.shared = it.seg >= g.E;
  const int local = item - t.prefix[it.seg];
  const int rows = t.rows[it.seg];
  const int rtiles = (rows + tile_rows - 1) / tile_rows;
  const int nt = local / rtiles;
  const int rt = local - nt * rtiles;
  // rtiles tiles of rows / rtiles rows, the first rows % rtiles of them one row more
  // (at most tile_rows each, as rows <= rtiles * tile_rows)
  const int base = rows / rtiles, extra = rows - base * rtiles;
  it.group = nt * groups_per_item;
  it.row0 = t.row0[it.seg] + rt * base + min(rt, extra);
  it.nrows = base + (rt < extra ? 1 : 0);
  return it;
}

}  // namespace afd
