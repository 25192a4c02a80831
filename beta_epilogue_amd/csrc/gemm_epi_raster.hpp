// gemm_epi_raster.hpp -- the order in which output tiles are handed out,
// shared by the GEMM kernel and the split-K reduction kernel so both agree on
// which tile a work item is.
//
// Within a batch the tiles run in a grouped raster: groups of `group_m` tile
// rows, and inside a group down the rows first, then across the columns, so
// tiles running at the same time share A row panels and B column panels in L2
// (the persistent tile loop of the Blackwell pipeline API card, "Device
// side").  Batches follow one another.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

struct TileRC {
  int l, tm, tn;  // batch, tile row, tile column
};

// Tile number ts (0 .. L*tiles_m*tiles_n - 1, below 2^31) in raster order.
__device__ __forceinline__ TileRC raster_tile(int ts, int tiles_m, int tiles_n, int group_m) {
  const unsigned tiles_mn = (unsigned)tiles_m * (unsigned)tiles_n;
  const int l = (int)((unsigned)ts / tiles_mn);
  const unsigned r = (unsigned)ts - (unsigned)l * tiles_mn;
  const unsigned gsize = (unsigned)group_m * (unsigned)tiles_n;
  const int gid = (int)(r / gsize);
  const int first_m = gid * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int within = (int)(r - (unsigned)gid * gsize);
  return TileRC{l, first_m + (int)((unsigned)within % (unsigned)gm), (int)((unsigned)within / (unsigned)gm)};
}

}  // namespace gemm_epi
