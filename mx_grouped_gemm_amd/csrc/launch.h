// Internal launchers (C++ linkage) called by the C-ABI layer in bsgemm_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

struct GemmArgs {
  const void* A;
  const void* a_scales;
  const void* B;
  const void* b_scales;
  const int32_t* expert_ids;    // nullptr: one dense group
  const int32_t* tile_offsets;  // nullptr: one dense group
  void* C;
  int M, N, K;
  int num_experts;
  int num_tiles;  // M-tiles of 128 rows to visit
  int num_cus;    // compute units of the device (size of a persistent grid)
  int group_m;    // blockwise work order: super-tiles per group (set by the launcher)
};

// Blockwise-FP8 (e4m3 x e4m3, fp32 1x128 / 128x128 scales). out: 1 f32, 2 bf16, 3 f16.
hipError_t launch_blockwise_fp8(const GemmArgs& a, int out, hipStream_t stream);

// Blockwise-FP8 with a workspace: with fewer work items than compute units each item is cut along
// K into ranges that run side by side (fp32 partial tiles and flags in ws; at most as many
// ranges as ws holds tiles). Falls back to launch_blockwise_fp8 when that does not apply.
hipError_t launch_blockwise_fp8_split(const GemmArgs& a, int out, void* ws, size_t ws_bytes, hipStream_t stream);

// Workspace bytes launch_blockwise_fp8_split needs on a device of num_cus compute units.
size_t blockwise_fp8_workspace_bytes(int num_cus);

// Blockwise-FP8 scheduled for M-tiles of few rows: one work item per M-tile x 256 columns.
hipError_t launch_blockwise_fp8_small_m(const GemmArgs& a, int out, hipStream_t stream);

// MX (e8m0 per 32 K). fmt_a / fmt_b: 1 e4m3, 2 e2m1. out: 1 f32, 2 bf16, 3 f16.
hipError_t launch_mx(const GemmArgs& a, int fmt_a, int fmt_b, int out, hipStream_t stream);

// nvfp4 (e2m1 x e2m1, e4m3 scale per 16 K; K a multiple of 256). out: 1 f32, 2 bf16, 3 f16.
hipError_t launch_nvfp4(const GemmArgs& a, int out, hipStream_t stream);

// Picks per expert (histogram of top-k ids).
hipError_t launch_route_counts(const int32_t* ids, int n, int E, int32_t* counts, hipStream_t stream);

// Rows of the picks in the grouped A, padding rows, and the e4m3 1x128 quantisation of the
// token rows into them. x_f32: 1 fp32 activations, 0 bf16.
hipError_t launch_quantize_permute(const void* x, int x_f32, const int32_t* ids, int tokens, int top_k,
                                   int K, int E, const int32_t* expert_offsets, int M, int32_t* dest,
                                   uint8_t* qa, float* a_scales, hipStream_t stream);

// Token-to-expert tile map.
hipError_t launch_build_tiles(const int32_t* counts, int num_experts, int num_tiles, int padded,
                              int32_t* expert_offsets, int32_t* tile_offsets, int32_t* expert_ids,
                              hipStream_t stream);

}  // namespace bsg
