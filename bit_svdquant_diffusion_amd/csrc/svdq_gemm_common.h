// Shared piece of the two GEMM kernels: the workgroup -> output-tile map.
#pragma once
#include "svdq_device.h"

namespace svdq {

struct TileMap {
  int tm, tn;
};
// Workgroup i runs on XCD i % 8. Give each XCD a contiguous range of tile
// indices, and walk tiles in groups of `group_m` tile-rows so that the
// workgroups resident on one XCD share A panels and B panels in its L2.
__device__ __forceinline__ TileMap map_tile(int bid, int tiles_m, int tiles_n, int group_m) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid & 7, j = bid >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + j;
  const int gsz = group_m * tiles_n;
  const int g = t / gsz;
  const int first = g * group_m;
  const int gm = min(tiles_m - first, group_m);
  const int in = t - g * gsz;
  return TileMap{first + in % gm, in / gm};
}

}  // namespace svdq
