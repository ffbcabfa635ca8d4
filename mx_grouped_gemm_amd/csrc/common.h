// Device helpers shared by the gfx950 kernels of the grouped block-scaled GEMM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS reads (and scalar loads) have completed: lgkmcnt(0), vmcnt and
// expcnt left at their maxima.
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier without the memory fence __syncthreads() adds (which would also wait for
// every outstanding prefetch). Callers wait for exactly the loads they need first.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ lds_void* as_lds(uint8_t* p) { return (lds_void*)p; }

// Raw buffer resource over [base, base + bytes): loads through it take a 32-bit per-lane offset
// (VGPR) plus a wave-uniform offset (SGPR), and reads past `bytes` return zero instead of
// touching memory. Word 3 selects 32-bit untyped data (gfx9 layout).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0xffffffffull ? (int)0xffffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Buffer -> LDS copies (buffer_load_dword{,x4} ... lds): lane i's bytes land at lds + i * size.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          lds_void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf2lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         lds_void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ v4i lds_read16(const uint8_t* p) { return *(const v4i*)p; }

__device__ __forceinline__ v8i cat(v4i lo, v4i hi) {
  return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// XOR swizzle of 16-byte chunks inside an LDS tile row of 128 bytes (8 chunks): chunk c of
// local row r is stored at slot c ^ swz8(r); 16 consecutive rows read at the same chunk then
// touch 16 different 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Column (within its 128-column block) held by LDS row l of a 128-row B tile half. Fragment j of a
// wave reads LDS rows 16 j .. 16 j + 15, and its MFMA gives lane (r16, q) the outputs of LDS rows
// 16 j + 4 q .. 16 j + 4 q + 3. Mapping row 16 j + 4 q + i to column 32 (j / 2) + 8 q + 4 (j % 2) + i
// gives the lane 8 consecutive columns in fragments 2 jj and 2 jj + 1: one 16-byte store of a
// bf16 / fp16 result, and the 4 lanes of a row cover 64 consecutive bytes.
__device__ __forceinline__ int b_col(int l) {
  const int j = l >> 4, q = (l >> 2) & 3, i = l & 3;
  return ((j >> 1) << 5) | (q << 3) | ((j & 1) << 2) | i;
}

// Output conversions (round to nearest even). A pair of fp32 values becomes one dword of two
// bf16 (gfx950 converts a pair in one instruction, v_cvt_pk_bf16_f32) or two fp16.
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t){lo, hi}, v2bf_t));
}
__device__ __forceinline__ uint32_t f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) { return f16_bits(lo) | (f16_bits(hi) << 16); }

enum OutKind { kOutF32 = 1, kOutBF16 = 2, kOutF16 = 3 };

// Store 4 consecutive fp32 values to C (row-major) at element offset `off` (a multiple of 4).
template <int OUT>
__device__ __forceinline__ void store4(void* C, size_t off, float a, float b, float c, float d) {
  if constexpr (OUT == kOutF32) {
    *(v4i*)((float*)C + off) = (v4i){(int)__float_as_uint(a), (int)__float_as_uint(b),
                                     (int)__float_as_uint(c), (int)__float_as_uint(d)};
  } else if constexpr (OUT == kOutBF16) {
    uint2 v;
    v.x = bf16x2_bits(a, b);
    v.y = bf16x2_bits(c, d);
    *(uint2*)((uint16_t*)C + off) = v;
  } else {
    uint2 v;
    v.x = f16x2_bits(a, b);
    v.y = f16x2_bits(c, d);
    *(uint2*)((uint16_t*)C + off) = v;
  }
}

// Store 8 consecutive fp32 values (lo, then hi) to C at element offset `off` (a multiple of 8):
// one 16-byte store for bf16 / fp16, two for fp32.
template <int OUT>
__device__ __forceinline__ void store8(void* C, size_t off, const float __attribute__((ext_vector_type(4))) & lo,
                                       const float __attribute__((ext_vector_type(4))) & hi) {
  if constexpr (OUT == kOutF32) {
    store4<OUT>(C, off, lo[0], lo[1], lo[2], lo[3]);
    store4<OUT>(C, off + 4, hi[0], hi[1], hi[2], hi[3]);
  } else {
    uint32_t (*cv)(float, float) = OUT == kOutBF16 ? bf16x2_bits : f16x2_bits;
    *(v4i*)((uint16_t*)C + off) = (v4i){(int)cv(lo[0], lo[1]), (int)cv(lo[2], lo[3]),
                                        (int)cv(hi[0], hi[1]), (int)cv(hi[2], hi[3])};
  }
}

// Work order. Blocks are dispatched round-robin over the 8 XCDs (each with its own L2), so
// block b runs on XCD b % 8. The grid is a multiple of 8 and block b takes logical item
// (b % 8) * (grid / 8) + b / 8: the blocks resident on one XCD work on consecutive logical
// items. Logical items walk groups of `group_m` M-tiles, column block by column block, so the
// items in flight on an XCD share A rows and B columns in its L2. Returns false for padding
// blocks past the last item.
__device__ __forceinline__ bool work_item(int num_tiles, int n_blocks, int group_m, int& t, int& nb) {
  const int grid = gridDim.x, b = blockIdx.x;
  const int L = (b % 8) * (grid / 8) + b / 8;
  if (L >= num_tiles * n_blocks) return false;
  const int per_group = group_m * n_blocks;
  const int g = L / per_group, r = L % per_group;
  const int t0 = g * group_m;
  const int gm = min(group_m, num_tiles - t0);
  nb = r / gm;
  t = t0 + r % gm;
  return true;
}

// Grid size for `items` work items: rounded up to a multiple of 8 (see work_item).
inline unsigned grid_for(long long items) { return (unsigned)((items + 7) / 8 * 8); }

// Work item of one M-tile: its expert and its row range [row0, row0 + rows).
struct TileRows {
  int expert, row0, rows;
};

// Resolve M-tile t (tile map or dense), clamping device-side contents into range.
__device__ __forceinline__ TileRows tile_rows(const int32_t* expert_ids, const int32_t* tile_offsets,
                                              int t, int M, int tile_m, int num_experts) {
  TileRows r;
  if (expert_ids) {
    r.expert = expert_ids[t];
    int a = tile_offsets[t], b = tile_offsets[t + 1];
    r.row0 = a;
    r.rows = min(max(b - a, 0), tile_m);
  } else {
    r.expert = 0;
    r.row0 = t * tile_m;
    r.rows = min(tile_m, M - r.row0);
  }
  if (r.expert < 0 || r.expert >= num_experts || r.row0 < 0 || r.row0 >= M) {
    r.rows = 0;
  } else {
    r.rows = min(r.rows, M - r.row0);
  }
  return r;
}

}  // namespace bsg
