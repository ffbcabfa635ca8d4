// Grouped blockwise-FP8 GEMM for gfx950 (MI355X).
//
// Computes, for every M-tile t of 128 rows with expert e = expert_ids[t], and every K block kb
// of 128 (the "k_iter" of the Modular MAX page "promote_accumulators", description paragraph
// and section Args; one promote per K iteration as in the page "EpilogueWarpContext",
// method per_k_stage):
//     P        = A[rows, kb] * B[e, cols, kb]^T            fp32 partial, started fresh
//     acc     += P * (a_scales[row, kb] * b_scales[e, col / 128, kb])
// then converts acc to the output type.
//
// CDNA4 mapping (not the pages' Blackwell design):
//  * block tile 256 (M) x 256 (N): two consecutive 128-row M-tiles of one expert (a lone tile,
//    or a pair whose experts differ, runs as one or two 128-row passes). The copy traffic per
//    flop of a 256 x 256 tile is two thirds of a 128 x 256 one. Measured by taking parts out:
//    the copies (their issue, not their latency), the promotion FMAs and the per-block barrier
//    each cost more than the LDS fragment reads.
//  * 8 waves (2 per SIMD), each owning 64 x 128 as 4 x 8 fragments of 16 x 16. One
//    v_mfma_scale_f32_16x16x128_f8f6f4 (scale operands neutral) computes a fragment's whole
//    128-wide K block, so the partial P is 4 registers and is promoted (4 FMAs) three MFMAs
//    after it was issued, by when it is mostly written (few wait states). Each MFMA, the
//    promotion that follows it and its LDS reads or copies form one scheduling region, so the
//    order is the source order. The 4 A fragments stay in registers for the K block, the 8 B
//    fragments stream through a 3-deep register queue two fragments ahead of their MFMAs.
//  * operands stream through a 2-stage LDS ring filled by buffer -> LDS copies
//    (buffer_load_dwordx4 ... lds); 16-byte chunks are XOR-swizzled so fragment reads are free
//    of bank conflicts. One barrier per K block, after the last read of the block's stage (in
//    pass 5 of 8) frees that stage for block b+2. A wave that issues a copy can stall at issue
//    while the CU's address unit works through the other waves' copies, so the 8 copies per
//    wave go out two per pass, each after an MFMA: B in passes 6 and 7 of block b, A (and the
//    B scales) in passes 0 and 1 of block b+1, all landing before the barrier of block b+1.
//  * A scales: each tile's rows are staged 8 K blocks at a time (256 rows x 8 floats, double
//    buffered), so a 128-byte line of the row-major a_scales serves 8 K blocks instead of one.
//    Column c of row r sits at slot c ^ ((r >> 3) & 7): the 16 rows one read instruction touches
//    (and the 4 rows of one lane) then fall in distinct banks.
//    The B scale of each of the two 128-column blocks rides in the stage.
//  * the MFMA computes C^T fragments (B rows as the first operand) so that each lane holds 4
//    consecutive output columns of one row: the epilogue writes 8-byte (bf16/fp16) or 16-byte
//    (fp32) vectors, and each lane needs one A scale per M fragment.
//  * in a pass of at most 192 (128, 64) rows, the waves whose 64 rows lie past the pass run the K
//    loop without reads, MFMAs or promotion, keeping only their copies, waits and barriers: a
//    lone 128-row tile then costs its SIMDs one wave's matrix work instead of two (the 8-expert
//    configuration, 8 such passes in 38, ran 12 % faster).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace bsg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128, TILE_M = 128;
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int WM = 64, WN = 128;                  // wave tile
constexpr int MI = WM / 16, NJ = WN / 16;         // 4 x 8 fragments of 16 x 16
constexpr int STAGES = 2;
constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;          // 32 KiB each per stage
constexpr int A_REGION = 0;
constexpr int B_REGION = STAGES * A_BYTES;                   // 64 KiB
constexpr int BS_REGION = B_REGION + STAGES * B_BYTES;       // 128 KiB: B scales, per stage
constexpr int BS_BYTES = 512;                                // 64 copies of each column block's scale
constexpr int AS_REGION = BS_REGION + STAGES * BS_BYTES;     // A scale chunks
constexpr int AS_CHUNK = 8;                                  // K blocks per A scale chunk
constexpr int AS_BYTES = BM * AS_CHUNK * 4;                  // 8 KiB per chunk
constexpr int LDS_BYTES = AS_REGION + 2 * AS_BYTES;          // 148480 of 160 KiB
constexpr int A_INSTR = A_BYTES / 1024 / NWAVES;             // 4
constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;             // 4
constexpr int AS_INSTR = AS_BYTES / 256 / NWAVES;            // 4 (4-byte copies, 64 lanes)
// forms of the K loop (see k_loop)
constexpr int MODE_IDLE = 0, MODE_FULL = 1, MODE_HALF = 2;

// Buffer resources of one unit of work (one pass of a work item over its rows): A rows, the
// expert's B rows of the column block, this wave's B scales and the A scales of the rows. A unit
// that does not exist gets resources of zero bytes: copies through them read zeros and touch no
// memory.
struct UnitRsrc {
  __amdgpu_buffer_rsrc_t a, b, bs, as;
};

// Per-lane parts of the copies. They depend only on the lane, the wave and K, so every unit of
// a workgroup shares them.
struct CopyPlan {
  uint32_t voff[A_INSTR];    // A copies: per-lane offset of instruction i
  uint32_t voff_b[B_INSTR];  // B copies: the same with B's rows permuted (see b_col)
  uint32_t as_vrow;          // A scale chunk: lane part of the row offset
  uint32_t as_row8;          // A scale chunk: bytes of 8 rows of a_scales
};

// LDS destinations are passed as 32-bit LDS addresses (wave base + constant): see LdsBases.
__device__ __forceinline__ lds_void* lds_ptr(uint32_t a) { return (lds_void*)(size_t)a; }

// Copy i (of A_INSTR / B_INSTR per wave) of K block kb to LDS address dst (the stage's A or B
// half plus this wave's part, see LdsBases), and the B scales of kb (waves 0 and 1, one column
// block each).
__device__ __forceinline__ void copy_a(uint32_t dst, __amdgpu_buffer_rsrc_t r, const CopyPlan& cp, int kb, int i) {
  buf2lds16(r, cp.voff[i], (uint32_t)__builtin_amdgcn_readfirstlane(kb) * BK, lds_ptr(dst + i * 1024));
}
__device__ __forceinline__ void copy_b(uint32_t dst, __amdgpu_buffer_rsrc_t r, const CopyPlan& cp, int kb, int i) {
  buf2lds16(r, cp.voff_b[i], (uint32_t)__builtin_amdgcn_readfirstlane(kb) * BK, lds_ptr(dst + i * 1024));
}
__device__ __forceinline__ void copy_bs(uint32_t dst, __amdgpu_buffer_rsrc_t r, int kb, int wave) {
  if (wave < 2) buf2lds4(r, 0, (uint32_t)__builtin_amdgcn_readfirstlane(kb) * 4, lds_ptr(dst));
}

__device__ __forceinline__ void issue_scale_chunk(uint32_t dst, __amdgpu_buffer_rsrc_t r,
                                                  const CopyPlan& cp, int chunk, int wave) {
  // Instruction i of wave w fills rows r = 32 w + 8 i + (lane >> 3); slot (lane & 7) of row r holds
  // column slot ^ ((r >> 1) & 7) = slot ^ (lane >> 4) ^ 4 (i & 1). Read by rows alone (16 rows 32
  // bytes apart, 4 lanes per row), the dword reads of a fragment's scales stalled the LDS on bank
  // conflicts (30.6M conflict cycles per gate_up launch of the 32-expert step); with this slot
  // order they take none (probed on gfx950 in isolation, and counted in the kernel). The per-lane
  // offsets are formed here from as_vrow (an empty asm keeps the compiler from hoisting all four
  // out of the loop).
  uint32_t v = cp.as_vrow + (uint32_t)__builtin_amdgcn_readfirstlane(chunk) * AS_CHUNK * 4;
  uint32_t sl = (threadIdx.x & 7) ^ ((threadIdx.x >> 4) & 3);
  asm volatile("" : "+v"(v), "+v"(sl));
#pragma unroll
  for (int i = 0; i < AS_INSTR; i++)
    buf2lds4(r, v + i * cp.as_row8 + ((sl ^ (4 * (i & 1))) << 2), 0, lds_ptr(dst + i * 256));
}

// This wave's LDS copy destinations: wb + region offset for A and B (a wave fills 4 KiB of each
// half), wbs for its B scale (waves 0 and 1), wch + buffer offset for its A scale rows. They are
// re-derived through an empty asm at every K block so that the compiler forms each destination
// (base + constant) next to its copy instead of keeping every combination live in SGPRs.
struct LdsBases {
  uint32_t wb, wbs, wch;
};

__device__ __forceinline__ LdsBases lds_bases(const uint8_t* smem, int wave) {
  const uint32_t s0 = (uint32_t)(size_t)as_lds(const_cast<uint8_t*>(smem));
  LdsBases l;
  l.wb = s0 + wave * A_INSTR * 1024;
  l.wbs = s0 + BS_REGION + wave * 256;
  l.wch = s0 + AS_REGION + wave * AS_INSTR * 256;
  asm volatile("" : "+s"(l.wb), "+s"(l.wbs), "+s"(l.wch));
  return l;
}

__device__ __forceinline__ v8i read_frag(const uint8_t* p, const int (&base)[2]) {
  return cat(lds_read16(p + base[0]), lds_read16(p + base[1]));
}

// The partial of one fragment: the unscaled fp8 MFMA (both format fields e4m3). The builtin is
// the scaled one; with both scale operands 0 the compiler emits v_mfma_f32_16x16x128_f8f6f4,
// which applies no scale and saves the scaled form's extra instruction word.
__device__ __forceinline__ v4f mma(const v8i& b, const v8i& a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                          0, 0, 0);
}


// Resources of unit u (zero bytes when !live): rows past the unit (ragged M), columns past N
// and scales past a_scales read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_a(const GemmArgs& p, const Unit& u, bool live) {
  const size_t K = (size_t)p.K;
  return make_rsrc((const uint8_t*)p.A + (size_t)u.row0 * K, live ? (uint64_t)u.rows * K : 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(const GemmArgs& p, const Unit& u, bool live) {
  const size_t K = (size_t)p.K;
  return make_rsrc((const uint8_t*)p.B + ((size_t)u.e * p.N + u.n0) * K,
                   live ? (uint64_t)min(BN, p.N - u.n0) * K : 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bs(const GemmArgs& p, const Unit& u, bool live, int wave) {
  const int N = p.N, KB = p.K / BK;
  const int cb = min(u.n0 / 128 + (wave & 1), N / 128 - 1);    // wave 0 / 1: column block 0 / 1
  return make_rsrc((const float*)p.b_scales + ((size_t)u.e * (N / 128) + cb) * KB, live ? (uint64_t)KB * 4 : 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_as(const GemmArgs& p, const Unit& u, bool live) {
  const int KB = p.K / BK;
  return make_rsrc((const float*)p.a_scales + (size_t)u.row0 * KB, live ? (uint64_t)u.rows * KB * 4 : 0);
}

// Workspace of the split schedule: one flag per (slot, pass) and an error word in the first 4 KiB,
// then one fp32 partial tile of 256 x 256 per slot. Slots are indexed by the cut between two
// workgroups' ranges, so a grid of G workgroups needs G + 1 slots at most.
constexpr size_t SPLIT_FLAG_BYTES = 4096;
constexpr int SPLIT_ERR_WORD = (int)(SPLIT_FLAG_BYTES / 4) - 1;
constexpr size_t SPLIT_SLOT_BYTES = (size_t)BM * BN * 4;
constexpr int SPLIT_SPIN_LIMIT = 1 << 22;   // about a second of s_sleep 8
// Cache policy of the partial tiles' buffer accesses: sc1, coherent at agent scope (the bits the
// compiler gives relaxed agent-scope atomics), so a partial written on one XCD is read from the
// coherence point on another without invalidating or writing back whole caches. The flags are
// relaxed agent-scope atomics; a writer waits for its partial's stores before its barrier and
// the flag store, a reader's partial loads are issued after it has seen the flag.
constexpr int SC_AGENT = 16;

struct SplitArgs {
  int items_dp;   // items [0, items_dp) are whole; the rest are split along K
  int parts;      // K ranges per split item (a power of 2, at most 16; 1: no item is split)
  uint8_t* ws;
  int* queue;     // whole items: 8 zeroed counters for the dynamic work order, or nullptr (static)
};

// Words of the workspace's first 4 KiB used by the launch of whole items: the dynamic order's 8
// counters (words 0-7), the counter of the last round's ranges (TAIL_CTR_WORD) and one flag per
// range from TAIL_FLAG_WORD0 on. A split launch uses words 0 .. items * parts - 1 as its flags.
constexpr int TAIL_CTR_WORD = 8;
constexpr int TAIL_FLAG_WORD0 = 16;
// Ranges of the last round's items have at least this many K blocks, and the last round is cut
// only in launches of fewer than TAIL_MAX_ROUNDS rounds of items. Measured over three jobs: the
// 8-expert workload (272 items, its last 16 in 8 ranges) 0.102-0.113 -> 0.096-0.101 ms; the
// 32-expert gate_up (33 rounds, its last 128 items in 2 ranges) 3.30-3.32 -> 3.30-3.35 ms: with
// many rounds the workgroups' whole items already end over a spread as wide as the ranges, which
// then only add their partial tiles' traffic.
constexpr int TAIL_MIN_KB = 4;
constexpr int TAIL_MAX_ROUNDS = 4;

// The dynamic work order (whole items, when the launch has a workspace): the grid's workgroups
// take the items of each XCD from a counter of that XCD instead of a fixed sequence. Items of at
// least this many K blocks use it (see the kernel's phase 1 and launch_blockwise_fp8_split).
constexpr int DYNAMIC_MIN_KB = 40;

// SPLIT: the split launch (items cut along K). LAST_RANGES (whole items): after its whole items,
// the workgroup takes ranges of the last round's items (see phase 2 below); a form of its own, so
// that launches without it keep the smaller kernel.
template <int OUT, bool SPLIT, bool LAST_RANGES>
__global__ __launch_bounds__(NTHREADS, 1) void bw_fp8_grouped_kernel(GemmArgs p, int n_blocks,
                                                                       const int32_t* __restrict__ expert_ids,
                                                                       const int32_t* __restrict__ tile_offsets,
                                                                       void* __restrict__ C, SplitArgs sp) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES + 16];   // + the work order's slot
  const TileMap tm = {expert_ids, tile_offsets};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int items = ((p.num_tiles + 1) / 2) * n_blocks;
  const int N = p.N, KB = p.K / BK;
  const size_t K = (size_t)p.K;
  const int wm = wave >> 1, wn = wave & 1;                  // rows 64 wm, cols 128 wn
  const int r16 = lane & 15, q = lane >> 4;
  // Consecutive K blocks of the units of this workgroup share one pipeline: the last blocks of a
  // unit copy the first blocks (and A scale chunks) of the next, so a unit after the first has
  // no prologue and its output stores drain under the next unit's first passes. This needs an
  // even number of K blocks (block 0 of every unit in stage 0); with an odd number each unit
  // starts with its own prologue.
  const bool piped = (KB & 1) == 0;
  const int nchunks = (KB + AS_CHUNK - 1) / AS_CHUNK;

  // Work order: the grid is a multiple of 8 and blocks are dispatched round-robin over the 8
  // XCDs, so block b runs on XCD b % 8. In each round of G = grid items, the blocks of one XCD
  // take a contiguous run of G / 8 items; items walk groups of group_m super-tiles column block by
  // column block, so the 32 items in flight on an XCD (4 super-tiles x 8 column blocks) share A
  // rows and B columns in its L2. (One super-tile across all its column blocks fetched a third
  // more beyond L2 and measured 3-9 % slower.)
  const int xb = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  // Without SPLIT: items [0, items_dp) as whole work items spread over the grid. With SPLIT: the
  // items from items_dp on, split along K over the whole grid (see the second phase below).
  const int items_dp = sp.items_dp;

  // per-lane LDS read bases: lane (r16, q) holds K bytes [32 q, 32 q + 32) of row r16 of a
  // fragment (two 16-byte chunks); the swizzle of row 16 f + r16 depends on r16 only
  const int sw = (r16 & 7) ^ ((r16 >> 3) & 1);
  int base_a[2], base_b[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int chunk = ((2 * q + h) ^ sw) * 16;
    base_a[h] = A_REGION + (wm * WM + r16) * BK + chunk;
    base_b[h] = B_REGION + (wn * WN + r16) * BK + chunk;
  }
  // A scale of row wm*64 + 16 i + r16, K block kb of a chunk: slot kb ^ ((r16 >> 1) & 7)
  static_assert(AS_REGION % 32 == 0, "scale rows must be 32-byte aligned");
  const int base_as = (AS_REGION + (wm * WM + r16) * AS_CHUNK * 4) | (((r16 >> 1) & 7) << 2);
  const int base_bs = BS_REGION + wn * 256;

  CopyPlan cp;
  {
    const int lrow = lane >> 3, slot = lane & 7;
    // Instruction i of wave w covers LDS rows 32 w + 8 i + lrow (swz8 of that row is
    // lrow ^ (i & 1)). The whole row offset sits in the per-lane offset, which the resource
    // bounds check.
#pragma unroll
    for (int i = 0; i < A_INSTR; i++) {
      const int l = wave * 32 + i * 8 + lrow;
      const uint32_t chunk = (uint32_t)((slot ^ lrow ^ (i & 1)) * 16);
      cp.voff[i] = (uint32_t)(l * K) + chunk;
      cp.voff_b[i] = (uint32_t)(((l & 128) | b_col(l & 127)) * K) + chunk;
    }
    // A scale chunk: instruction i of wave w covers rows 32 w + 8 i + lrow
    cp.as_vrow = (uint32_t)((wave * 32 + lrow) * KB * 4);
    cp.as_row8 = (uint32_t)(8 * KB * 4);
  }

  int cbase = 0;   // A scale buffer of the current unit's first chunk; chunk c0 + r is in buffer (cbase + r) & 1
  // The copy resources. Piped, each switches from the current unit to the next at the block
  // from which its copies only target the next unit (B: block KB-2, A and B scales: KB-1,
  // A scales: the block that loads the next unit's first chunk), so at a unit's start they
  // already describe it.
  UnitRsrc rc;
  v4f acc[MI][NJ];

  // The K loop of unit u over its blocks [kb0, kend) into acc. prologue: copy the unit's first two
  // blocks and A scale chunks and wait for the first (else the previous unit's last blocks copied
  // them). pipe: the last two blocks copy the first blocks of unit nx (zero-byte resources unless
  // nx_live), which must then start at block 0; needs kend - kb0 even.
  auto run_unit = [&](const Unit& u, const int kb0, const int kend, const bool prologue, const bool pipe,
                      const Unit& nx, const bool nx_live, const bool half) {
    const int rows = u.rows;
    const int nb = kend - kb0;
    const int c0 = kb0 / AS_CHUNK, cl = (kend - 1) / AS_CHUNK;   // first and last chunk of the unit
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (prologue) {
      // A scales of chunks c0 and c0 + 1, block kb0 and the B half of block kb0 + 1 (its A half and
      // B scales go out in passes 0 and 1 of block kb0, as in every block); block kb0 published
      cbase = 0;
      rc.a = rsrc_a(p, u, true);
      rc.b = rsrc_b(p, u, true);
      rc.bs = rsrc_bs(p, u, true, wave);
      rc.as = rsrc_as(p, u, true);
      const LdsBases lb = lds_bases(smem, wave);
      issue_scale_chunk(lb.wch, rc.as, cp, c0, wave);
      issue_scale_chunk(lb.wch + AS_BYTES, rc.as, cp, c0 + 1, wave);
#pragma unroll
      for (int i = 0; i < A_INSTR; i++) copy_a(lb.wb + A_REGION, rc.a, cp, kb0, i);
#pragma unroll
      for (int i = 0; i < B_INSTR; i++) copy_b(lb.wb + B_REGION, rc.b, cp, kb0, i);
      copy_bs(lb.wbs, rc.bs, kb0, wave);
#pragma unroll
      for (int i = 0; i < B_INSTR; i++) copy_b(lb.wb + B_REGION + B_BYTES, rc.b, cp, min(kb0 + 1, kend - 1), i);
      wait_vmcnt<0>();
      barrier();
    }

      // The K loop, in three forms (MODE). FULL: the wave's 64 x 128 of a pass of more than 128
      // rows. IDLE: a wave with nothing to compute (its rows lie past the pass) runs the loop
      // without reads, MFMAs or promotion. HALF: a pass of at most 128 rows is split over the 8
      // waves as 2 x 4 tiles of 64 x 64 (rows 64 (w / 4), columns 64 (w % 4)), so each SIMD keeps
      // two waves of matrix work instead of one. Every form issues the same copies at the same
      // points and reaches every barrier, so all keep one sequence of waits and barriers.
      auto k_loop = [&](auto mode_tag) {
      constexpr int MODE = decltype(mode_tag)::value;
      constexpr bool ACT = MODE != MODE_IDLE;
      constexpr int SL = MODE == MODE_HALF ? 2 : MI;    // MFMA slots per pass (8 passes per block)
      constexpr int NK = 8 * SL;                        // MFMAs per block
      // per-lane LDS read bases of this form (HALF: formed here and made opaque, so that they are
      // not kept live through the other forms)
      int ba[2], bb[2], bas;
      int bbs = base_bs;
      if constexpr (MODE == MODE_HALF) {
        const int hm = wave >> 2, hq = wave & 3;
  #pragma unroll
        for (int h = 0; h < 2; h++) {
          const int chunk = ((2 * q + h) ^ sw) * 16;
          ba[h] = A_REGION + (hm * WM + r16) * BK + chunk;
          bb[h] = B_REGION + ((hq >> 1) * 128 + (hq & 1) * 64 + r16) * BK + chunk;
        }
        bas = (AS_REGION + (hm * WM + r16) * AS_CHUNK * 4) | (((r16 >> 1) & 7) << 2);
        bbs = BS_REGION + (hq >> 1) * 256;
        asm volatile("" : "+v"(ba[0]), "+v"(ba[1]), "+v"(bb[0]), "+v"(bb[1]), "+v"(bas));
      } else {
        ba[0] = base_a[0];
        ba[1] = base_a[1];
        bb[0] = base_b[0];
        bb[1] = base_b[1];
        bas = base_as;
      }
      v8i af[MI], bq[3];
      float as_raw[MI], bs_raw = 0.f;
      if constexpr (ACT) {
  #pragma unroll
        for (int i = 0; i < MI; i++) af[i] = read_frag(smem + i * 2048, ba);
        bq[0] = read_frag(smem, bb);
        bq[1] = read_frag(smem + 2048, bb);
        const int as0 = (bas ^ ((kb0 % AS_CHUNK) * 4)) + (cbase & 1) * AS_BYTES;
  #pragma unroll
        for (int i = 0; i < MI; i++) as_raw[i] = *(const float*)(smem + as0 + i * 16 * AS_CHUNK * 4);
        bs_raw = *(const float*)(smem + bbs);
      }

      // One K block (kb, the r-th of the unit). S (its stage) is a constant so every LDS offset is
      // an immediate. Blocks of the main loop (TAIL false) copy from the current unit only; the last
      // two blocks (TAIL true) copy the next unit's first blocks when piped, else repeat block
      // kend-1 into a stage that is not read again. MFMA k of a block multiplies B fragment k / MI
      // by A fragment k % MI (FULL: 8 B fragments over 8 passes of 4; HALF: 4 over 8 passes of 2).
      auto k_block = [&](auto stage_tag, auto tail_tag, const int r) {
        const int b = kb0 + r;
        constexpr int S = decltype(stage_tag)::value;
        constexpr bool TAIL = decltype(tail_tag)::value;
        constexpr int so_ab = S * A_BYTES, sn_ab = (S ^ 1) * A_BYTES;   // this and the other stage
        constexpr int sn_bs = (S ^ 1) * BS_BYTES;
        // copy targets: the A half and B scales of block b+1, the B half of block b+2
        int kb_a = b + 1, kb_b = min(b + 2, kend - 1);
        if constexpr (TAIL) {
          if (pipe) {
            kb_b = b + 2 - kend;
            if (b == kend - 1) {
              kb_a = 0;
              rc.a = rsrc_a(p, nx, nx_live);
              rc.bs = rsrc_bs(p, nx, nx_live, wave);
            }
          } else {
            kb_a = min(b + 1, kend - 1);
          }
        }
        const LdsBases lb = lds_bases(smem, wave);
        float sc[MI];
        if constexpr (ACT) {
  #pragma unroll
          for (int i = 0; i < MI; i++) sc[i] = as_raw[i] * bs_raw;
        }
        v4f part[4];
        // the MFMA of slot k, and the promotion of the partial three slots back (pinned there,
        // which also keeps the MFMAs in their pass)
        auto mfma_slot = [&](const int k) {
          part[k % 4] = mma(bq[(k / MI) % 3], af[k % MI]);
          if (k >= 3) {
            const int kp = k - 3, jp = kp / MI, ip = kp % MI;
            acc[ip][jp] += part[kp % 4] * sc[ip];
            asm volatile("" : "+v"(acc[ip][jp]));
          }
        };
        // passes 0..5 at raised wave priority so the SIMD's arbiter favours feeding the matrix
        // unit. Reads of the B fragments two ahead (FULL: fragment j + 2 in two halves, after the
        // first and the third MFMA of pass j; HALF: fragments 2 and 3 in passes 0 and 2). Passes 0
        // and 1 also copy the A half and B scales of block b+1 into the other stage (freed by the
        // barrier of block b-1; its B half went out in passes 6 and 7 of block b-1), two copies per
        // pass.
  #pragma unroll
        for (int j = 0; j < 6; j++) {
          __builtin_amdgcn_sched_barrier(0);
          v4i lo, hi;
          __builtin_amdgcn_s_setprio(1);
  #pragma unroll
          for (int i = 0; i < SL; i++) {
            if constexpr (ACT) mfma_slot(j * SL + i);
            if (j < 2 && (MODE == MODE_HALF || (i & 1))) {
              copy_a(lb.wb + A_REGION + sn_ab, rc.a, cp, kb_a, MODE == MODE_HALF ? 2 * j + i : 2 * j + (i >> 1));
              if (j == 1 && i == SL - 1) copy_bs(lb.wbs + sn_bs, rc.bs, kb_a, wave);
            }
            if constexpr (MODE == MODE_FULL) {
              if (j + 2 < NJ && i == 0) lo = lds_read16(smem + so_ab + (j + 2) * 2048 + bb[0]);
              if (j + 2 < NJ && i == 2) hi = lds_read16(smem + so_ab + (j + 2) * 2048 + bb[1]);
            } else if constexpr (MODE == MODE_HALF) {
              if ((j == 0 || j == 2) && i == 0) lo = lds_read16(smem + so_ab + (j / 2 + 2) * 2048 + bb[0]);
              if ((j == 0 || j == 2) && i == 1) hi = lds_read16(smem + so_ab + (j / 2 + 2) * 2048 + bb[1]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_setprio(0);
          if constexpr (MODE == MODE_FULL) {
            if (j + 2 < NJ) bq[(j + 2) % 3] = cat(lo, hi);
          } else if constexpr (MODE == MODE_HALF) {
            if (j == 0 || j == 2) bq[(j / 2 + 2) % 3] = cat(lo, hi);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // This wave's reads of stage S are done and its copies of block b+1 have landed; after
        // the barrier every wave's have, so block b+1 is readable and stage S is free.
        wait_vmcnt<0>();
        wait_lds_reads();
        barrier();
        if constexpr (TAIL) {
          if (pipe && b == kend - 2) rc.b = rsrc_b(p, nx, nx_live);
        }
        __builtin_amdgcn_sched_barrier(0);
        // pass 6 (no reads left in this block) with copies 0 and 1 of the B half of block b+2 into
        // stage S; HALF: the MFMAs of pass 6 are the last of A fragments 0 and 1, which are
        // refilled from block b+1 right after them
  #pragma unroll
        for (int i = 0; i < SL; i++) {
          if constexpr (ACT) {
            mfma_slot(6 * SL + i);
            if constexpr (MODE == MODE_HALF) af[i] = read_frag(smem + sn_ab + i * 2048, ba);
          }
          if (MODE == MODE_HALF || (i & 1)) copy_b(lb.wb + B_REGION + so_ab, rc.b, cp, kb_b, MODE == MODE_HALF ? i : i >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // A scale chunks. Chunk c (blocks 8c .. 8c+7) goes into its buffer in block 8(c-1), when
        // the buffer's previous chunk (c-2) has been read by every wave. A unit's first two chunks
        // are loaded before it starts: in its prologue, or piped in the previous unit's blocks
        // kend-2 and kend-1 (the first chunk's buffer held chunk n-2 of that unit, n = its chunk
        // count, and the second's its last chunk, read for the last time before the barrier of
        // block kend-1). Whole units start at block 0, so in them only even blocks begin a chunk.
        if constexpr (!TAIL && (SPLIT || S == 0)) {
          if (b % AS_CHUNK == 0 && b > kb0 && b / AS_CHUNK + 1 <= cl) {
            const int c = b / AS_CHUNK + 1;
            issue_scale_chunk(lb.wch + ((cbase + c - c0) & 1) * AS_BYTES, rc.as, cp, c, wave);
          }
        }
        if constexpr (TAIL) {
          if (pipe && b == kend - 2) {
            rc.as = rsrc_as(p, nx, nx_live);
            issue_scale_chunk(lb.wch + ((cbase + cl - c0 + 1) & 1) * AS_BYTES, rc.as, cp, 0, wave);
          }
          if (pipe && b == kend - 1)
            issue_scale_chunk(lb.wch + ((cbase + cl - c0) & 1) * AS_BYTES, rc.as, cp, 1, wave);
        }
        __builtin_amdgcn_sched_barrier(0);
        // pass 7: the last MFMAs of the other A fragments (all four in FULL), each refilled from
        // block b+1 right after its MFMA, then the first two B fragments and the scales of block
        // b+1 are read; copies 2 and 3 of the B half of block b+2.
  #pragma unroll
        for (int i = 0; i < SL; i++) {
          if constexpr (ACT) {
            const int k = 7 * SL + i;
            mfma_slot(k);
            af[k % MI] = read_frag(smem + sn_ab + (k % MI) * 2048, ba);
          }
          if (MODE == MODE_HALF || (i & 1))
            copy_b(lb.wb + B_REGION + so_ab, rc.b, cp, kb_b, MODE == MODE_HALF ? 2 + i : 2 + (i >> 1));
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ACT) {
          bq[0] = read_frag(smem + sn_ab, bb);
          bq[1] = read_frag(smem + sn_ab + 2048, bb);
          const int bn = min(b + 1, kend - 1);
          const int as_v = (bas ^ ((bn % AS_CHUNK) * 4)) + ((cbase + bn / AS_CHUNK - c0) & 1) * AS_BYTES;
  #pragma unroll
          for (int i = 0; i < MI; i++)
            as_raw[i] = *(const float*)(smem + as_v + i * 16 * AS_CHUNK * 4);
          bs_raw = *(const float*)(smem + sn_bs + bbs);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the last three partials of the block
        if constexpr (ACT) {
  #pragma unroll
          for (int k = NK - 3; k < NK; k++) {
            const int jp = k / MI, ip = k % MI;
            acc[ip][jp] += part[k % 4] * sc[ip];
            asm volatile("" : "+v"(acc[ip][jp]));
          }
        }
      };

      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      int r = 0;
      for (; r + 2 < nb; r += 2) {
        k_block(S0{}, std::false_type{}, r);
        k_block(S1{}, std::false_type{}, r + 1);
      }
      // nb even: the unit's last two blocks (stages 0 and 1); nb odd: its last block (stage 0)
      k_block(S0{}, std::true_type{}, r);
      if (r + 1 < nb) k_block(S1{}, std::true_type{}, r + 1);
      };
      if (half && rows <= TILE_M) {
        if ((wave >> 2) * WM < rows)
          k_loop(std::integral_constant<int, MODE_HALF>{});
        else
          k_loop(std::integral_constant<int, MODE_IDLE>{});
      } else if (wm * WM < rows) {
        k_loop(std::integral_constant<int, MODE_FULL>{});
      } else {
        k_loop(std::integral_constant<int, MODE_IDLE>{});
      }

  };

  // epilogue: lane holds row r16 of each M fragment and, over N fragments 2 jj and 2 jj + 1,
  // columns 32 jj + 8 q .. 32 jj + 8 q + 7 of its 128-column block (see b_col); in the HALF form
  // (a pass of at most 128 rows) the wave's 64 columns start at 128 (w % 4 / 2) + 64 (w % 2) and
  // its rows at 64 (w / 4). The stores are not waited for: the next unit's first wait before a
  // barrier covers them.
  auto store_c = [&](const Unit& u, const bool half) {
    const int hm = half ? wave >> 2 : wm;
    const int cw = half ? ((wave & 3) >> 1) * 128 + (wave & 1) * 64 : wn * WN;
    const int nf = half ? 2 : NJ / 2;
#pragma unroll
    for (int i = 0; i < MI; i++) {
      const int mloc = hm * WM + i * 16 + r16;
      if (mloc >= u.rows) continue;
      const size_t crow = (size_t)(u.row0 + mloc) * N;
#pragma unroll
      for (int jj = 0; jj < NJ / 2; jj++) {
        const int col = u.n0 + cw + jj * 32 + q * 8;
        if (jj < nf && col < N) store8<OUT>(C, crow + col, acc[i][2 * jj], acc[i][2 * jj + 1]);
      }
    }
  };

  // Sum share jp of an item's partial tiles, slots slot0 .. slot0 + P - 1, in slot order and store
  // it: v4f entries [jp * PER, (jp + 1) * PER) of the 8 x 32 x 64 in a tile, entry jp * PER +
  // k * 512 + tid for thread tid. Entry g is lane g % 64 of fragment (g / 64) % 32 of wave slot
  // g / 2048 (pass ws / 4 of a two-pass item, else pass 0), as the waves wrote them. All of a
  // thread's loads are issued before the first sum, so the share costs one memory latency.
  auto reduce_share = [&](auto parts_tag, const Unit* u, const int np, const int slot0, const int jp) {
    constexpr int P = decltype(parts_tag)::value;
    constexpr int ENTRIES = 8 * MI * NJ * kWave;
    constexpr int PER = ENTRIES / P;
    constexpr int EPT = PER / NTHREADS;   // entries per thread
    static_assert(PER % NTHREADS == 0, "a share is whole rows of threads");
    const __amdgpu_buffer_rsrc_t all =
        make_rsrc(sp.ws + SPLIT_FLAG_BYTES + (size_t)slot0 * SPLIT_SLOT_BYTES, (uint64_t)P * SPLIT_SLOT_BYTES);
    v4f v[EPT][P];
#pragma unroll
    for (int k = 0; k < EPT; k++)
#pragma unroll
      for (int m = 0; m < P; m++)
        v[k][m] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                              all, (uint32_t)(jp * PER + k * NTHREADS + tid) * 16,
                                              (uint32_t)(m * SPLIT_SLOT_BYTES), SC_AGENT));
#pragma unroll
    for (int k = 0; k < EPT; k++) {
      const int g = jp * PER + k * NTHREADS + tid;
      const int wsl = g / (MI * NJ * kWave), idx = (g / kWave) % (MI * NJ), ln = g % kWave;
      const int ps = np == 2 ? wsl >> 2 : 0;
      const int vw = np == 2 ? wsl & 3 : wsl;          // the wave that held the entry
      const Unit& w = ps == 0 ? u[0] : u[1];
      const int fi = idx / NJ, fj = idx % NJ;
      const int mloc = (vw >> 1) * WM + fi * 16 + (ln & 15);
      const int col = w.n0 + (vw & 1) * WN + ((fj >> 1) << 5) + ((ln >> 4) << 3) + ((fj & 1) << 2);
      if (ps >= np || mloc >= w.rows || col >= N) continue;
      v4f sum = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < P; m++) sum += v[k][m];
      store4<OUT>(C, (size_t)(w.row0 + mloc) * N + col, sum[0], sum[1], sum[2], sum[3]);
    }
  };

  // Range jp of item L cut along K into `parts` ranges of blocks: run it (never piped, never HALF;
  // the caller has passed a barrier after the workgroup's last LDS reads), write the fp32 partial
  // tile to slot slot0 + jp of the workspace, raise flags[slot0 + jp], wait until the item's
  // `parts` flags are up, then sum share jp (a 1/parts slice of the tile) over the item's
  // partials and store it to C. The wait ends after a bounded number of polls, should a part
  // ever not run, and then sets the workspace's error word (the item's output is then wrong, and
  // reported, rather than hung).
  auto split_part = [&](const int L, const int jp, const int parts, const int slot0, int* const flags) {
    const int kb0 = jp * KB / parts, kend = (jp + 1) * KB / parts;
    const int slot = slot0 + jp;
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(sp.ws + SPLIT_FLAG_BYTES + (size_t)slot * SPLIT_SLOT_BYTES, SPLIT_SLOT_BYTES);
    Unit u[2];
    const int np = __builtin_amdgcn_readfirstlane(item_units(p, tm, n_blocks, L, u));
    for (int ps = 0; ps < np; ps++) {
      Unit w = ps == 0 ? u[0] : u[1];
      w.e = __builtin_amdgcn_readfirstlane(w.e);
      w.row0 = __builtin_amdgcn_readfirstlane(w.row0);
      w.rows = __builtin_amdgcn_readfirstlane(w.rows);
      w.n0 = __builtin_amdgcn_readfirstlane(w.n0);
      if (ps > 0) barrier();   // every wave is past its last LDS read of the previous pass
      run_unit(w, kb0, kend, true, false, w, false, false);
      // partial tile: per (wave, pass) 32 x 1 KiB, lane-contiguous; a pass of an item of two
      // passes has at most 128 rows (waves 0-3), so its second pass uses waves 4-7's space
      if (wm * WM < w.rows) {
        const uint32_t pv = (uint32_t)(((wave + 4 * ps) * (MI * NJ * kWave) + lane) * 16);
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
          for (int j = 0; j < NJ; j++)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc[i][j]), pr, pv,
                                                   (i * NJ + j) * kWave * 16, SC_AGENT);
      }
    }
    wait_vmcnt<0>();   // this wave's partial has reached the agent's coherence point
    barrier();
    if (tid == 0) {
      __hip_atomic_store(flags + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int m = 0; m < parts; m++) {
        int spins = 0;
        while (__hip_atomic_load(flags + slot0 + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
          if (++spins > SPLIT_SPIN_LIMIT) {   // never expected: give up, record it, go on
            __hip_atomic_store((int*)sp.ws + SPLIT_ERR_WORD, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
      }
    }
    barrier();
    switch (parts) {
      case 2: reduce_share(std::integral_constant<int, 2>{}, u, np, slot0, jp); break;
      case 4: reduce_share(std::integral_constant<int, 4>{}, u, np, slot0, jp); break;
      case 8: reduce_share(std::integral_constant<int, 8>{}, u, np, slot0, jp); break;
      default: reduce_share(std::integral_constant<int, 16>{}, u, np, slot0, jp); break;
    }
  };

  // Phase 1 (not SPLIT): whole items below items_dp, one pipeline through all. Static order: items
  // xb, xb + G, ... With sp.queue, the dynamic order: the XCD's items in the same order (round r
  // of the static order gives XCD x items r G + x G/8 .. r G + x G/8 + G/8 - 1), but each
  // workgroup takes the XCD's next one from the XCD's counter when it needs one. In the static
  // order a workgroup that meets slower items (two passes) falls behind the others of its XCD for
  // good, and the items in flight on the XCD then share less in its L2; the counters keep them
  // together. Thread 0 asks for the next item one item ahead, so its answer has long arrived when
  // it is used; a barrier passes it to the workgroup through LDS.
  if constexpr (!SPLIT) {
    UnitSeq seq;
    seq.L = xb - (int)gridDim.x;
    seq.k = 0;
    int* const queue = sp.queue;
    const int xcd = blockIdx.x % 8, G8 = gridDim.x / 8;
    if (queue) seq.L = -1;
    int pending = 0;
    // the counter's address goes through an opaque per-lane zero so that the compiler keeps the
    // single-lane atomic as it is (a wave-aggregated form would need its result at once)
    int zero = 0;
    asm volatile("" : "+v"(zero));
    typedef __attribute__((address_space(3))) int lds_int;
    lds_int* const slot = (lds_int*)(smem + LDS_BYTES);
    if (queue && tid == 0) pending = __hip_atomic_fetch_add(queue + xcd + zero, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    auto take = [&](const int v, UnitSeq& q) {
      q.L = (v / G8) * (int)gridDim.x + xcd * G8 + v % G8;
      q.k = 0;
    };
    // Take the item thread 0 asked for last time and ask for the next one. Counter values are
    // taken in increasing order, so once a taken item lies past the last, so does every later one.
    auto grab = [&](UnitSeq& q) {
      barrier();   // every wave has read the slot's previous value
      if (tid == 0) {
        *slot = pending;
        pending = __hip_atomic_fetch_add(queue + xcd + zero, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_lds_reads();
      barrier();
      take(__builtin_amdgcn_readfirstlane(*slot), q);
    };
    auto next = [&](UnitSeq& q, Unit& out) -> bool {
      if (!queue) return next_unit(p, tm, n_blocks, items_dp, q, out);
      Unit u[2];
      int n = q.L < 0 ? 0 : item_units(p, tm, n_blocks, q.L, u);
      if (q.k >= n) {
        grab(q);   // the answer asked for one item ago has long arrived
        if (q.L >= items_dp) return false;
        n = item_units(p, tm, n_blocks, q.L, u);
        while (n == 0) {   // an item without a live tile: take the next (here it may be waited for)
          grab(q);
          if (q.L >= items_dp) return false;
          n = item_units(p, tm, n_blocks, q.L, u);
        }
      }
      out = q.k == 0 ? u[0] : u[1];
      q.k++;
      out.e = __builtin_amdgcn_readfirstlane(out.e);
      out.row0 = __builtin_amdgcn_readfirstlane(out.row0);
      out.rows = __builtin_amdgcn_readfirstlane(out.rows);
      out.n0 = __builtin_amdgcn_readfirstlane(out.n0);
      return true;
    };
    Unit cu, nx;
    bool have = next(seq, cu);
    bool have_next = have && next(seq, nx);
    for (bool first = true; have; first = false) {
      if (!first && !piped) barrier();   // every wave is past its last LDS read of the previous unit
      const bool half = cu.rows <= TILE_M;
      run_unit(cu, 0, KB, first || !piped, piped, nx, have_next && piped, half);
      store_c(cu, half);
      if (!have_next) break;
      cbase = (cbase + nchunks) & 1;
      cu = nx;
      have_next = next(seq, nx);
    }

    // Phase 2 (LAST_RANGES): the last round's items [items_dp, items), fewer than the grid, each
    // cut along K into sp.parts ranges. A workgroup that has run out of whole items takes the next
    // range from one counter, so the ranges go to the workgroups that finish first and the grid
    // ends together instead of a few workgroups running a whole item more. Ranges are taken in
    // counter order, so the ranges an item's parts wait for have been or will be taken by
    // workgroups that are running.
    if constexpr (LAST_RANGES) {
      const int parts = sp.parts;
      const int nranges = (items - items_dp) * parts;
      int* const words = (int*)sp.ws;
      for (;;) {
        barrier();   // every wave is past its last LDS read, of the ring and of the slot
        if (tid == 0) *slot = __hip_atomic_fetch_add(words + TAIL_CTR_WORD + zero, 1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        wait_lds_reads();
        barrier();
        const int r = __builtin_amdgcn_readfirstlane(*slot);
        if (r >= nranges) break;
        split_part(items_dp + r / parts, r % parts, parts, r / parts * parts, words + TAIL_FLAG_WORD0);
      }
    }
  }

  // Phase 2 (SPLIT, a launch of its own): the items [items_dp, items) (all of them; fewer than the
  // grid). Each is cut along K into sp.parts ranges run side by side by workgroups parts * t ..
  // parts * t + parts - 1 (consecutive, so on one XCD), flags in words 0 .. items * parts - 1 of
  // the workspace, cleared on the stream before the launch. The grid is one workgroup per compute
  // unit, and an item's parts are consecutive workgroups that start together, so the parts a
  // workgroup waits for are running.
  if constexpr (SPLIT) {
    const int parts = sp.parts;
    const int t = xb / parts, jp = xb % parts;
    if (items_dp + t >= items) return;
    split_part(items_dp + t, jp, parts, t * parts, (int*)sp.ws);
  }
}

}  // namespace

namespace {

__global__ void zero_words_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int OUT, bool SPLIT, bool LAST_RANGES>
hipError_t launch_out(const GemmArgs& a, int n_blocks, unsigned grid, SplitArgs sp, hipStream_t stream) {
  hipLaunchKernelGGL((bw_fp8_grouped_kernel<OUT, SPLIT, LAST_RANGES>), dim3(grid), dim3(NTHREADS), 0, stream, a, n_blocks,
                     a.expert_ids, a.tile_offsets, a.C, sp);
  return hipGetLastError();
}

template <bool SPLIT, bool LAST_RANGES = false>
hipError_t launch(const GemmArgs& a0, int out, int n_blocks, unsigned grid, SplitArgs sp, hipStream_t stream) {
  GemmArgs a = a0;
  // Super-tiles per group of the work order (see the kernel): 4, so that an XCD's 32 items in
  // flight are 4 super-tiles x 8 column blocks (32-expert step, alternating runs on one box:
  // groups of 2 / 4 / 8 / 16 super-tiles 5.286 / 5.197 / 5.214 / 5.360 ms); with at most 8
  // column blocks, 1 (4 super-tiles x 8 column blocks as well), which measured 10-15 % faster
  // than 8 on the 8-expert N = 2048 workload.
  a.group_m = n_blocks <= 8 ? 1 : 4;
  switch (out) {
    case kOutF32: return launch_out<kOutF32, SPLIT, LAST_RANGES>(a, n_blocks, grid, sp, stream);
    case kOutBF16: return launch_out<kOutBF16, SPLIT, LAST_RANGES>(a, n_blocks, grid, sp, stream);
    case kOutF16: return launch_out<kOutF16, SPLIT, LAST_RANGES>(a, n_blocks, grid, sp, stream);
    default: return hipErrorInvalidValue;
  }
}

// Workgroups of the split schedule's grid: whole multiples of 8 (XCD order), one per compute unit.
unsigned split_grid(int num_cus) { return (unsigned)(num_cus / 8 * 8); }


}  // namespace

hipError_t launch_blockwise_fp8(const GemmArgs& a, int out, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long items = (long long)((a.num_tiles + 1) / 2) * n_blocks;
  if (items == 0) return hipSuccess;
  if (items > 0x7ffffff0LL) return hipErrorInvalidValue;
  // persistent grid: one workgroup per compute unit (the LDS ring allows one), fewer when there
  // are fewer items; a multiple of 8 for the XCD-aware order
  const unsigned grid = grid_for(items < a.num_cus ? items : a.num_cus);
  return launch<false>(a, out, n_blocks, grid, SplitArgs{(int)items, 1, nullptr, nullptr}, stream);
}

size_t blockwise_fp8_workspace_bytes(int num_cus) {
  return SPLIT_FLAG_BYTES + (size_t)split_grid(num_cus) * SPLIT_SLOT_BYTES;
}

hipError_t launch_blockwise_fp8_split(const GemmArgs& a, int out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long items = (long long)((a.num_tiles + 1) / 2) * n_blocks;
  const unsigned G = split_grid(a.num_cus);
  const int KB = a.K / BK;
  if (items == 0) return hipSuccess;
  if (items > 0x7ffffff0LL) return hipErrorInvalidValue;
  // With fewer items than workgroups, each item is cut along K into `parts` ranges (a power of
  // 2, at most 16, each at least 8 K blocks), as many as the grid holds.
  // A workspace smaller than blockwise_fp8_workspace_bytes (at least the flags) holds fewer
  // partial tiles; the split then uses fewer ranges, so that every range has its tile.
  if (ws == nullptr || ws_bytes < SPLIT_FLAG_BYTES) return hipErrorInvalidValue;
  const long long slots = std::min<long long>(G, (long long)((ws_bytes - SPLIT_FLAG_BYTES) / SPLIT_SLOT_BYTES));
  const long long tail = items < (long long)G ? items : 0;
  int parts = 1;
  while (tail > 0 && parts < 16 && 2 * parts * 8 <= KB && tail * 2 * parts <= slots) parts *= 2;
  const int words = (int)(SPLIT_FLAG_BYTES / 4);
  if (parts < 2 || G > SPLIT_FLAG_BYTES / 4 - 1) {
    if (items < (long long)G) return launch_blockwise_fp8(a, out, stream);
    // Whole items, in one launch with two additions that need the workspace:
    // * items of DYNAMIC_MIN_KB or more K blocks take the dynamic work order (8 counters).
    //   Measured on the 32-expert workload in one job: gate_up (56 K blocks) 3.48 -> 3.33 ms,
    //   while down (16 K blocks, whose workgroups change items more often, so that the XCD's
    //   items in flight straddle two rounds' runs more often) went 1.81 -> 1.88 ms and the
    //   8-expert one (32 K blocks) did not change;
    // * in a launch of fewer than TAIL_MAX_ROUNDS rounds, the last round's items (items % G of
    //   them) are cut along K into tparts ranges (a power of 2, at most 16, each at least
    //   TAIL_MIN_KB blocks, as many as the grid and the workspace hold) that the workgroups which
    //   run out of whole items first take from a counter.
    const bool dyn = KB >= DYNAMIC_MIN_KB;
    const long long last = items % G;
    int tparts = 1;
    while (last > 0 && items < (long long)TAIL_MAX_ROUNDS * G && tparts < 16 && KB >= 2 * tparts * TAIL_MIN_KB &&
           last * 2 * tparts <= slots && TAIL_FLAG_WORD0 + last * 2 * tparts < SPLIT_ERR_WORD)
      tparts *= 2;
    if (!dyn && tparts < 2) return launch_blockwise_fp8(a, out, stream);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream, (int*)ws, words);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (tparts < 2) return launch<false>(a, out, n_blocks, G, SplitArgs{(int)items, 1, nullptr, (int*)ws}, stream);
    return launch<false, true>(a, out, n_blocks, G,
                               SplitArgs{(int)(items - last), tparts, (uint8_t*)ws, dyn ? (int*)ws : nullptr}, stream);
  }
  hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream, (int*)ws, words);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch<true>(a, out, n_blocks, G, SplitArgs{0, parts, (uint8_t*)ws, nullptr}, stream);
}

}  // namespace bsg
