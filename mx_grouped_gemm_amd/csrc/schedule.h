// Work distribution of the persistent 256 x 256 GEMM kernels (blockwise FP8 and MX): work items,
// their passes, and the sequence of passes ("units") a workgroup runs.
#pragma once

#include "common.h"
#include "launch.h"

namespace bsg {

constexpr int kTileM = 128;   // rows of an M-tile of the tile map
constexpr int kItemN = 256;   // columns of a work item

// The tile map, from kernel arguments declared __restrict__ so that the compiler may read it with
// scalar loads (counted apart from the copies in flight, which a vector load's wait would drain).
struct TileMap {
  const int32_t* expert_ids;
  const int32_t* tile_offsets;
};

// One pass of a work item: rows [row0, row0 + rows) of expert e against columns [n0, n0 + 256).
struct Unit {
  int e, row0, rows, n0;
};

// The passes of work item L (super-tile L / n_blocks, column block L % n_blocks): one 256-row pass
// when its two 128-row tiles are consecutive full rows of one expert, else one pass per live tile.
// Returns the number of passes (0 when both tiles are skipped).
__device__ __forceinline__ int item_units(const GemmArgs& p, const TileMap& tm, int n_blocks, int L, Unit (&u)[2]) {
  // groups of p.group_m super-tiles walk their column blocks together (one super-tile per step)
  const int gsz = p.group_m * n_blocks, g0 = (L / gsz) * p.group_m;
  const int gm = min(p.group_m, (p.num_tiles + 1) / 2 - g0), r = L % gsz;
  const int s = g0 + r % gm, n0 = (r / gm) * kItemN;
  const TileRows t0 = tile_rows(tm.expert_ids, tm.tile_offsets, 2 * s, p.M, kTileM, p.num_experts);
  TileRows t1 = {0, 0, 0};
  if (2 * s + 1 < p.num_tiles)
    t1 = tile_rows(tm.expert_ids, tm.tile_offsets, 2 * s + 1, p.M, kTileM, p.num_experts);
  u[0] = {t0.expert, t0.row0, t0.rows, n0};
  u[1] = {t1.expert, t1.row0, t1.rows, n0};
  if (t0.rows == kTileM && t1.rows > 0 && t1.expert == t0.expert && t1.row0 == t0.row0 + kTileM) {
    u[0].rows = kTileM + t1.rows;
    return 1;
  }
  if (t0.rows > 0) return t1.rows > 0 ? 2 : 1;
  u[0] = u[1];
  return t1.rows > 0 ? 1 : 0;
}

// The units of one workgroup, in order: items xb, xb + G, xb + 2 G, ... (G = grid size), each
// item's passes in turn. L is the current item, k the index of the next pass to take from it.
struct UnitSeq {
  int L, k;
};

__device__ __forceinline__ bool next_unit(const GemmArgs& p, const TileMap& tm, int n_blocks, int items,
                                          UnitSeq& q, Unit& out) {
  Unit u[2];
  int n = q.L < 0 ? 0 : item_units(p, tm, n_blocks, q.L, u);
  while (q.k >= n) {
    q.L += gridDim.x;
    if (q.L >= items) return false;
    n = item_units(p, tm, n_blocks, q.L, u);
    q.k = 0;
  }
  out = q.k == 0 ? u[0] : u[1];
  q.k++;
  out.e = __builtin_amdgcn_readfirstlane(out.e);
  out.row0 = __builtin_amdgcn_readfirstlane(out.row0);
  out.rows = __builtin_amdgcn_readfirstlane(out.rows);
  out.n0 = __builtin_amdgcn_readfirstlane(out.n0);
  return true;
}

}  // namespace bsg
