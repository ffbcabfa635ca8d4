// Token-to-expert tile map: per-expert row counts -> expert row offsets, per-M-tile row
// offsets and per-M-tile expert ids (the group bookkeeping that the "expert_ids" and
// "scheduler" arguments of the Modular MAX page "promote_accumulators" presuppose).
//
// Every block recomputes the (small) exclusive scans over the experts in LDS, then handles a
// grid-strided share of the tiles; a tile finds its expert by binary search over the tile
// prefix. Block 0 also writes expert_offsets.
#include "common.h"
#include "launch.h"

namespace bsg {

constexpr int kMapThreads = 256;
constexpr int kMaxExperts = 4096;
constexpr int kTileM = 128;

__global__ __launch_bounds__(kMapThreads) void build_tiles_kernel(
    const int32_t* __restrict__ counts, int E, int T, int padded, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ tile_offsets, int32_t* __restrict__ expert_ids) {
  __shared__ long long row_start[kMaxExperts + 1];  // first row of expert e
  __shared__ int tile_start[kMaxExperts + 1];       // first tile of expert e
  __shared__ long long part_rows[kMapThreads];
  __shared__ int part_tiles[kMapThreads];

  const int tid = threadIdx.x;
  // each thread scans a contiguous chunk of experts
  const int per = (E + kMapThreads - 1) / kMapThreads;
  const int lo = min(tid * per, E), hi = min(lo + per, E);
  long long rsum = 0;
  int tsum = 0;
  for (int e = lo; e < hi; e++) {
    int c = max(counts[e], 0);
    int tiles = (c + kTileM - 1) / kTileM;
    rsum += padded ? (long long)tiles * kTileM : (long long)c;
    tsum += tiles;
  }
  part_rows[tid] = rsum;
  part_tiles[tid] = tsum;
  __syncthreads();
  // inclusive Hillis-Steele scan over the per-thread partials
  for (int d = 1; d < kMapThreads; d <<= 1) {
    long long r = tid >= d ? part_rows[tid - d] : 0;
    int t = tid >= d ? part_tiles[tid - d] : 0;
    __syncthreads();
    part_rows[tid] += r;
    part_tiles[tid] += t;
    __syncthreads();
  }
  long long rbase = tid ? part_rows[tid - 1] : 0;
  int tbase = tid ? part_tiles[tid - 1] : 0;
  for (int e = lo; e < hi; e++) {
    row_start[e] = rbase;
    tile_start[e] = tbase;
    int c = max(counts[e], 0);
    int tiles = (c + kTileM - 1) / kTileM;
    rbase += padded ? (long long)tiles * kTileM : (long long)c;
    tbase += tiles;
  }
  if (tid == kMapThreads - 1) {
    row_start[E] = part_rows[kMapThreads - 1];
    tile_start[E] = part_tiles[kMapThreads - 1];
  }
  __syncthreads();

  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kMapThreads) expert_offsets[e] = (int32_t)row_start[e];
  }
  const int used = tile_start[E];
  const long long total_rows = row_start[E];
  for (int t = blockIdx.x * kMapThreads + tid; t <= T; t += gridDim.x * kMapThreads) {
    int e = -1;
    long long start = total_rows;
    if (t < used) {
      // largest e with tile_start[e] <= t (empty experts share their successor's start)
      int a = 0, b = E;  // invariant: tile_start[a] <= t < tile_start[b]
      while (b - a > 1) {
        int mid = (a + b) >> 1;
        if (tile_start[mid] <= t) a = mid; else b = mid;
      }
      e = a;
      start = row_start[e] + (long long)(t - tile_start[e]) * kTileM;
    }
    if (padded) start = (long long)t * kTileM;
    tile_offsets[t] = (int32_t)start;
    if (t < T) expert_ids[t] = e;
  }
}

hipError_t launch_build_tiles(const int32_t* counts, int num_experts, int num_tiles, int padded,
                              int32_t* expert_offsets, int32_t* tile_offsets, int32_t* expert_ids,
                              hipStream_t stream) {
  int blocks = (num_tiles + 1 + kMapThreads - 1) / kMapThreads;
  blocks = blocks < 1 ? 1 : (blocks > 64 ? 64 : blocks);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(blocks), dim3(kMapThreads), 0, stream, counts,
                     num_experts, num_tiles, padded, expert_offsets, tile_offsets, expert_ids);
  return hipGetLastError();
}

}  // namespace bsg
