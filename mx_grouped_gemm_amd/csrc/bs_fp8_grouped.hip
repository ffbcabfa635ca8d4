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
//  * block = 8 waves (2 per SIMD), tile 128 (M) x 256 (N); each wave owns 64 x 64 as 2 x 2
//    fragments of 32 x 32. A 128-wide K block is two v_mfma_scale_f32_32x32x64_f8f6f4 (scale
//    operands neutral), one per 64-wide K half, chained into a fresh fp32 partial P in VGPRs;
//    the promote is 16 FMAs per lane per fragment into VGPR accumulators.
//  * ping-pong schedule: waves 0-3 (group 0, rows 0-63) and 4-7 (group 1, rows 64-127) put one
//    wave of each group on every SIMD and run half a K block out of phase around the single
//    barrier per K block. Group 0 issues the MFMAs of block b, passes barrier b, then promotes
//    b and reads block b+1; group 1 promotes b-1 and reads b, passes barrier b, then issues
//    the MFMAs of b. Between two barriers each SIMD holds one wave feeding the matrix unit and
//    one wave doing the VALU promotion and LDS reads, and the two overlap.
//  * operands stream through a 3-stage LDS ring filled by buffer -> LDS copies
//    (buffer_load_dwordx4 ... lds) that group 0 issues three K blocks ahead; 16-byte chunks are
//    XOR-swizzled so fragment reads are free of bank conflicts. The scales ride in the same
//    ring: 128 A scales (one per row) and the block's B scales (one per 128 columns).
//  * the MFMA computes C^T fragments (B rows as the first operand) so that each lane holds 4
//    consecutive output columns of one row: the epilogue writes 8-byte (bf16/fp16) or 16-byte
//    (fp32) vectors.
#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int NCOPY = 4;                                    // waves issuing the copies (group 0)
constexpr int WAVE_M = 64, WAVE_N = 64;                     // wave tile: 2 x 2 fragments
constexpr int FM = WAVE_M / 32, FN = WAVE_N / 32;
constexpr int STAGES = 3;
constexpr int A_BYTES = BM * BK;                            // 16 KiB
constexpr int B_BYTES = BN * BK;                            // 32 KiB
// scale strip: copy wave w owns 64 floats at SS_OFF + 256 w; floats 0..31 are the A scales of
// rows 32w..32w+31 and float 32 is the B scale of the 64-column block w (of its 128 columns)
constexpr int SS_OFF = A_BYTES + B_BYTES;
constexpr int SS_BYTES = NCOPY * 64 * 4;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SS_BYTES;   // 50176
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;             // 150528 of 160 KiB
constexpr int A_INSTR = A_BYTES / 1024 / NCOPY;             // 1 KiB copies per copy wave
constexpr int B_INSTR = B_BYTES / 1024 / NCOPY;
constexpr int LOADS_PER_STAGE = A_INSTR + B_INSTR + 2;      // + A-scale and B-scale copies

// Per-thread copy plan of one stage (lane i of a 1 KiB instruction covers row i/8, 16-byte
// slot i%8 of that row). Sources are buffer resources over the block's rows (wave-uniform,
// scalar registers) plus 32-bit per-lane offsets; a K block advances the scalar offset only.
// Rows past the tile (ragged M) or past N read as zero through the resource bounds.
struct LoadPlan {
  __amdgpu_buffer_rsrc_t a_rsrc;   // A rows of the tile
  __amdgpu_buffer_rsrc_t b_rsrc;   // B[e] rows of the column block
  __amdgpu_buffer_rsrc_t as_rsrc;  // a_scales rows of the tile
  __amdgpu_buffer_rsrc_t bs_rsrc;  // b_scales[e] row of this wave's 64-column block
  uint32_t a_off[A_INSTR], b_off[B_INSTR], as_off;
  int a_dst[A_INSTR], b_dst[B_INSTR], ss_dst;
};


// Fragment read offsets inside a stage.
struct FragPlan {
  int a_off[FM][2][2];  // [m fragment][K half][16-byte half]
  int b_off[FN][2][2];  // [n fragment][K half][16-byte half]
  int as_off[FM];       // A scale of the lane's row, per m fragment
  int bs_off;           // B scale of the wave's column block
};

// Fragments of one K block: both 64-wide halves, 32 bytes per lane per fragment half.
struct Frags {
  v8i a[FM][2];
  v8i b[FN][2];
};

// The stage's scales for this lane, kept raw: the product is formed where it is used.
struct Scales {
  float a[FM];
  float b;
};

__device__ __forceinline__ void issue_stage(uint8_t* dst, const LoadPlan& lp, int kb, int lane) {
  kb = __builtin_amdgcn_readfirstlane(kb);                     // uniform: scalar offsets
  const uint32_t koff = (uint32_t)kb * BK, soff = (uint32_t)kb * 4;
#pragma unroll
  for (int i = 0; i < A_INSTR; i++) buf2lds16(lp.a_rsrc, lp.a_off[i], koff, as_lds(dst + lp.a_dst[i]));
#pragma unroll
  for (int i = 0; i < B_INSTR; i++) buf2lds16(lp.b_rsrc, lp.b_off[i], koff, as_lds(dst + lp.b_dst[i]));
  if (lane < 32) buf2lds4(lp.as_rsrc, lp.as_off, soff, as_lds(dst + lp.ss_dst));
  if (lane == 32) buf2lds4(lp.bs_rsrc, 0, soff, as_lds(dst + lp.ss_dst));
}

// Read one K half (kh) of the block's fragments from a stage.
__device__ __forceinline__ void read_half(const uint8_t* st, const FragPlan& fp, int kh, Frags& f) {
#pragma unroll
  for (int i = 0; i < FM; i++)
    f.a[i][kh] = cat(lds_read16(st + fp.a_off[i][kh][0]), lds_read16(st + fp.a_off[i][kh][1]));
#pragma unroll
  for (int j = 0; j < FN; j++)
    f.b[j][kh] = cat(lds_read16(st + fp.b_off[j][kh][0]), lds_read16(st + fp.b_off[j][kh][1]));
}

__device__ __forceinline__ void read_frags(const uint8_t* st, const FragPlan& fp, Frags& f) {
  read_half(st, fp, 0, f);
  read_half(st, fp, 1, f);
}

__device__ __forceinline__ void read_scales(const uint8_t* st, const FragPlan& fp, Scales& sc) {
  sc.b = *(const float*)(st + fp.bs_off);
#pragma unroll
  for (int i = 0; i < FM; i++) sc.a[i] = *(const float*)(st + fp.as_off[i]);
}

// The K block's fresh partial of every fragment: the two K halves chained.
__device__ __forceinline__ void mma_block(const Frags& f, v16f (&part)[FM][FN]) {
  const v16f zero = (v16f){};
#pragma unroll
  for (int mi = 0; mi < FM; mi++)
#pragma unroll
    for (int ni = 0; ni < FN; ni++)
      part[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[ni][0], f.a[mi][0], zero,
                                                                    0, 0, 0, 127, 0, 127);
#pragma unroll
  for (int mi = 0; mi < FM; mi++)
#pragma unroll
    for (int ni = 0; ni < FN; ni++)
      part[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[ni][1], f.a[mi][1],
                                                                    part[mi][ni], 0, 0, 0, 127,
                                                                    0, 127);
  // keep the MFMAs in this phase (not sunk past the barrier to their use)
#pragma unroll
  for (int mi = 0; mi < FM; mi++)
#pragma unroll
    for (int ni = 0; ni < FN; ni++) asm volatile("" : "+v"(part[mi][ni]));
}

__device__ __forceinline__ void promote(const v16f (&part)[FM][FN], const Scales& sc,
                                        v16f (&acc)[FM][FN]) {
#pragma unroll
  for (int mi = 0; mi < FM; mi++) {
    const float s = sc.a[mi] * sc.b;
#pragma unroll
    for (int ni = 0; ni < FN; ni++) acc[mi][ni] += part[mi][ni] * s;
  }
}

// Wait until this wave's copies of the stage about to be published have landed: the copies of
// the following K block (if issued) may stay in flight.
__device__ __forceinline__ void wait_vmcnt_for(bool following_in_flight) {
  if (following_in_flight) wait_vmcnt<LOADS_PER_STAGE>(); else wait_vmcnt<0>();
}

// Refill order. A fragment register may only be overwritten once the MFMAs reading it have
// finished, or the LDS read stalls on them. The first-half MFMAs of a block are issued first,
// so the first-half registers are refilled first; the second half is refilled after the
// promotion, which itself waits for all of this wave's MFMAs to complete.

// Group 0, K block b: MFMAs of b (operands in f); barrier b (its copies of stage b+1 have
// landed, its reads of stage b are done); copies of block b+3 into stage b's slot; refill the
// first half from block b+1; promote b; refill the second half. `next_st` (stage b+1) and
// `cur_st` (stage b) are distinct: __restrict__ lets the compiler keep the copies into cur_st
// in flight across the reads of next_st (their completion is awaited before a later barrier).
__device__ __forceinline__ void step_g0(const uint8_t* __restrict__ next_st, uint8_t* __restrict__ cur_st,
                                        const LoadPlan& lp, const FragPlan& fp, int lane, int b,
                                        int KB, Frags& f, Scales& sc, v16f (&acc)[FM][FN]) {
  v16f part[FM][FN];
  mma_block(f, part);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt_for(b + 2 < KB);
  wait_lds_reads();
  barrier();
  if (b + 3 < KB) issue_stage(cur_st, lp, b + 3, lane);
  __builtin_amdgcn_sched_barrier(0);
  const Scales s_b = sc;
  const bool more = b + 1 < KB;
  if (more) {
    read_half(next_st, fp, 0, f);
    read_scales(next_st, fp, sc);
  }
  __builtin_amdgcn_sched_barrier(0);
  promote(part, s_b, acc);
  __builtin_amdgcn_sched_barrier(0);
  if (more) read_half(next_st, fp, 1, f);
}

// Group 1, K block b: refill the first half from block b (stage published at barrier b-1);
// promote b-1 (partials in part); refill the second half; barrier b (its reads of stage b are
// done); MFMAs of b. Group 1 issues no copies.
__device__ __forceinline__ void step_g1(const uint8_t* st_b, const FragPlan& fp, int b, Frags& f,
                                        Scales& sc, v16f (&part)[FM][FN], v16f (&acc)[FM][FN]) {
  const Scales s_prev = sc;
  read_half(st_b, fp, 0, f);
  read_scales(st_b, fp, sc);
  __builtin_amdgcn_sched_barrier(0);
  if (b > 0) promote(part, s_prev, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_half(st_b, fp, 1, f);
  __builtin_amdgcn_sched_barrier(0);
  wait_lds_reads();
  barrier();
  __builtin_amdgcn_sched_barrier(0);
  mma_block(f, part);
}

template <int OUT>
__global__ __launch_bounds__(NTHREADS, 1) void bw_fp8_grouped_kernel(GemmArgs p, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int t, nb;
  if (!work_item(p.num_tiles, n_blocks, 8, t, nb)) return;
  const int n0 = nb * BN;
  const TileRows tr = tile_rows(p.expert_ids, p.tile_offsets, t, p.M, BM, p.num_experts);
  if (tr.rows <= 0) return;
  // the tile's expert and rows are block-uniform: keep them in scalar registers
  const int e = __builtin_amdgcn_readfirstlane(tr.expert);
  const int row0 = __builtin_amdgcn_readfirstlane(tr.row0);
  const int rows = __builtin_amdgcn_readfirstlane(tr.rows);
  const int N = p.N, KB = p.K / BK;
  const size_t K = (size_t)p.K;
  const uint8_t* A = (const uint8_t*)p.A;
  const uint8_t* Be = (const uint8_t*)p.B + (size_t)e * N * K;
  const float* a_scales = (const float*)p.a_scales;
  const float* b_scales = (const float*)p.b_scales;
  const bool group0 = wave < NCOPY;
  const int wm = wave >> 2, wn = wave & 3;                     // rows 64 wm, cols 64 wn
  const int ncols = min(BN, N - n0);

  // ---- copy plan (group 0 only) ----
  LoadPlan lp;
  if (group0) {
    lp.a_rsrc = make_rsrc(A + (size_t)row0 * K, (uint64_t)rows * K);
    lp.b_rsrc = make_rsrc(Be + (size_t)n0 * K, (uint64_t)ncols * K);
    lp.as_rsrc = make_rsrc(a_scales + (size_t)row0 * KB, (uint64_t)rows * KB * 4);
    const int nb = min((n0 + wave * WAVE_N) / 128, N / 128 - 1);
    lp.bs_rsrc = make_rsrc(b_scales + ((size_t)e * (N / 128) + nb) * KB, (uint64_t)KB * 4);
    const int lrow = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int i = 0; i < A_INSTR; i++) {                        // wave w: A rows [32w, 32w+32)
      const int r = (wave * A_INSTR + i) * 8 + lrow;
      lp.a_off[i] = (uint32_t)(r * K + (slot ^ swz8(r)) * 16);
      lp.a_dst[i] = (wave * A_INSTR + i) * 8 * BK;
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; i++) {                        // wave w: B rows [64w, 64w+64)
      const int r = (wave * B_INSTR + i) * 8 + lrow;
      lp.b_off[i] = (uint32_t)(r * K + (slot ^ swz8(r)) * 16);
      lp.b_dst[i] = A_BYTES + (wave * B_INSTR + i) * 8 * BK;
    }
    lp.as_off = (uint32_t)((wave * 32 + (lane & 31)) * KB * 4);
    lp.ss_dst = SS_OFF + wave * 64 * 4;
  }

  // ---- fragment read plan ----
  FragPlan fp;
  const int fr = lane & 31, kq = lane >> 5;
#pragma unroll
  for (int kh = 0; kh < 2; kh++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int c = kh * 4 + kq * 2 + j;                       // 16-byte K chunk of this lane
#pragma unroll
      for (int f = 0; f < FM; f++) {
        const int ra = wm * WAVE_M + f * 32 + fr;
        fp.a_off[f][kh][j] = ra * BK + ((c ^ swz8(ra)) * 16);
      }
#pragma unroll
      for (int f = 0; f < FN; f++) {
        const int rb = wn * WAVE_N + f * 32 + fr;
        fp.b_off[f][kh][j] = A_BYTES + rb * BK + ((c ^ swz8(rb)) * 16);
      }
    }
#pragma unroll
  for (int f = 0; f < FM; f++) {
    const int ra = wm * WAVE_M + f * 32 + fr;
    fp.as_off[f] = SS_OFF + (ra >> 5) * 256 + (ra & 31) * 4;
  }
  fp.bs_off = SS_OFF + wn * 256 + 32 * 4;

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = (v16f){};

  // prologue: group 0 puts K blocks 0, 1, 2 in flight; stage 0 published; group 0 holds block 0
  if (group0) {
    issue_stage(smem, lp, 0, lane);
    if (KB > 1) issue_stage(smem + STAGE_BYTES, lp, 1, lane);
    if (KB > 2) issue_stage(smem + 2 * STAGE_BYTES, lp, 2, lane);
    if (KB > 2) wait_vmcnt<2 * LOADS_PER_STAGE>();
    else wait_vmcnt_for(KB > 1);
  }
  barrier();
  Frags f;
  Scales sc;
  if (group0) {
    read_frags(smem, fp, f);
    read_scales(smem, fp, sc);
    for (int b = 0; b < KB; b++)
      step_g0(smem + ((b + 1) % STAGES) * STAGE_BYTES, smem + (b % STAGES) * STAGE_BYTES, lp, fp,
              lane, b, KB, f, sc, acc);
  } else {
    v16f part[FM][FN];
    for (int b = 0; b < KB; b++)
      step_g1(smem + (b % STAGES) * STAGE_BYTES, fp, b, f, sc, part, acc);
    promote(part, sc, acc);
  }

  // ---- epilogue: lane holds row (fr) and columns 8g + 4kq + {0..3} of each fragment ----
#pragma unroll
  for (int mi = 0; mi < FM; mi++) {
    const int mloc = wm * WAVE_M + mi * 32 + fr;
    if (mloc >= rows) continue;
    const size_t crow = (size_t)(row0 + mloc) * N;
#pragma unroll
    for (int ni = 0; ni < FN; ni++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int col = n0 + wn * WAVE_N + ni * 32 + g * 8 + kq * 4;
        if (col < N)
          store4<OUT>(p.C, crow + col, acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1],
                      acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
      }
  }
}

}  // namespace

hipError_t launch_blockwise_fp8(const GemmArgs& a, int out, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long blocks = (long long)a.num_tiles * n_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0LL) return hipErrorInvalidValue;
  dim3 grid(grid_for(blocks)), block(NTHREADS);
  switch (out) {
    case kOutF32: hipLaunchKernelGGL(bw_fp8_grouped_kernel<kOutF32>, grid, block, 0, stream, a, n_blocks); break;
    case kOutBF16: hipLaunchKernelGGL(bw_fp8_grouped_kernel<kOutBF16>, grid, block, 0, stream, a, n_blocks); break;
    case kOutF16: hipLaunchKernelGGL(bw_fp8_grouped_kernel<kOutF16>, grid, block, 0, stream, a, n_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsg
