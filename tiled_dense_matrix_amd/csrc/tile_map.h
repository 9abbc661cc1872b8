// Device helpers shared by the tiled kernels: mapping a workgroup id to an
// output tile (one workgroup owns one tile of C, CS336 Lecture 5 GPU notes,
// §4.2) in an order that keeps neighbouring tiles on one XCD.
#pragma once

#include <hip/hip_runtime.h>

namespace tdm {

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// and each XCD has a private L2. Renumber the ids so that XCD x owns one
// contiguous run of tile numbers, then walk tiles in groups of `group_m`
// tile-rows (column-major inside a group), so tiles that share rows of A or
// columns of B run on the same XCD at the same time.
__device__ __forceinline__ void xcd_tile(int bid, int tiles_m, int tiles_n,
                                         int group_m, int& tm, int& tn) {
  constexpr int kXcds = 8;
  const int total = tiles_m * tiles_n;
  int t = bid;
  if (total % kXcds == 0) t = (bid % kXcds) * (total / kXcds) + bid / kXcds;
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int rows = min(tiles_m - first_m, group_m);
  const int r = t - g * per_group;
  tm = first_m + r % rows;
  tn = r / rows;
}

}  // namespace tdm
