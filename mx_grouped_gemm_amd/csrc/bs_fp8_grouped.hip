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
//    operands neutral) chained into a fresh fp32 partial P in VGPRs; the promote is 16 FMAs per
//    lane per fragment into VGPR accumulators. The other wave on the SIMD fills the matrix
//    unit while one wave promotes.
//  * operands stream through a 3-stage LDS ring filled by direct global->LDS loads
//    (global_load_lds_dwordx4), 16-byte chunks XOR-swizzled so fragment reads are free of
//    bank conflicts. The scales of a stage ride in the same ring: 128 A scales (one per row)
//    and the block's two B scales (one per 128 columns; a wave's 64 columns sit inside one
//    128-column block, so its B scale is a broadcast read).
//  * the MFMA computes C^T fragments (B rows as the first operand) so that each lane holds 4
//    consecutive output columns of one row: the epilogue writes 8-byte (bf16/fp16) or 16-byte
//    (fp32) vectors.
#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int STAGES = 3;
constexpr int A_BYTES = BM * BK;                            // 16 KiB
constexpr int B_BYTES = BN * BK;                            // 32 KiB
// scale strip: wave w owns 32 floats at SS_OFF + 128 w; floats 0..15 are the A scales of rows
// 16w..16w+15, and wave 0's floats 16, 17 are the B scales of the block's two column blocks
constexpr int SS_OFF = A_BYTES + B_BYTES;
constexpr int SS_BYTES = NWAVES * 32 * 4;
constexpr int BS_OFF = SS_OFF + 16 * 4;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SS_BYTES;   // 50176
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;             // 150528 of 160 KiB
constexpr int LOADS_PER_STAGE = 2 + 4 + 1;                  // per wave: A, B, scales

// Per-thread global -> LDS copy plan of one stage (lane i of a 1 KiB instruction covers row
// i/8, 16-byte slot i%8 of that row).
struct LoadPlan {
  const uint8_t* a_src[2];
  const uint8_t* b_src[4];
  const float* ss_src;  // this lane's scale row (advances by one float per K block)
  int a_dst[2], b_dst[4], ss_dst;
  bool ss_lane;
};

// Fragment read offsets inside a stage.
struct FragPlan {
  int a_off[2][2][2];  // [m fragment][K half][16-byte half]
  int b_off[2][2][2];  // [n fragment][K half][16-byte half]
  int as_off[2];       // A scale of the lane's row, per m fragment
  int bs_off;          // B scale of the wave's column block
};

// Issue the global -> LDS copies of K block kb into stage `dst`.
__device__ __forceinline__ void issue_stage(uint8_t* dst, const LoadPlan& lp, int kb) {
  const size_t koff = (size_t)kb * BK;
#pragma unroll
  for (int i = 0; i < 2; i++) g2lds16(lp.a_src[i] + koff, as_lds(dst + lp.a_dst[i]));
#pragma unroll
  for (int i = 0; i < 4; i++) g2lds16(lp.b_src[i] + koff, as_lds(dst + lp.b_dst[i]));
  if (lp.ss_lane) g2lds4(lp.ss_src + kb, as_lds(dst + lp.ss_dst));
}

// One K block: issue the copies of K block `kb_next` into `nxt` (if requested), then multiply
// the operands resident in `cur` and promote into acc. `cur` and `nxt` are distinct stages;
// marking them __restrict__ lets the compiler keep the copies in flight across the LDS reads
// (their completion is awaited explicitly before the next barrier).
__device__ __forceinline__ void bw_step(const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt,
                                        const LoadPlan& lp, const FragPlan& fp, bool issue,
                                        int kb_next, v16f (&acc)[2][2]) {
  if (issue) issue_stage(nxt, lp, kb_next);
  v8i af[2][2], bf[2][2];
#pragma unroll
  for (int f = 0; f < 2; f++)
#pragma unroll
    for (int kh = 0; kh < 2; kh++) {
      af[f][kh] = cat(lds_read16(cur + fp.a_off[f][kh][0]), lds_read16(cur + fp.a_off[f][kh][1]));
      bf[f][kh] = cat(lds_read16(cur + fp.b_off[f][kh][0]), lds_read16(cur + fp.b_off[f][kh][1]));
    }
  const float bs = *(const float*)(cur + fp.bs_off);
  float sc[2];
#pragma unroll
  for (int f = 0; f < 2; f++) sc[f] = *(const float*)(cur + fp.as_off[f]) * bs;
  const v16f zero = (v16f){};
#pragma unroll
  for (int mi = 0; mi < 2; mi++)
#pragma unroll
    for (int ni = 0; ni < 2; ni++) {
      v16f part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[ni][0], af[mi][0], zero,
                                                                 0, 0, 0, 127, 0, 127);
      part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[ni][1], af[mi][1], part,
                                                            0, 0, 0, 127, 0, 127);
      acc[mi][ni] += part * sc[mi];                            // promote
    }
}

template <int OUT>
__global__ __launch_bounds__(NTHREADS, 1) void bw_fp8_grouped_kernel(GemmArgs p, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x / n_blocks;
  const int n0 = (blockIdx.x % n_blocks) * BN;
  const TileRows tr = tile_rows(p.expert_ids, p.tile_offsets, t, p.M, BM, p.num_experts);
  if (tr.rows <= 0) return;
  const int e = tr.expert, row0 = tr.row0, rows = tr.rows;
  const int N = p.N, KB = p.K / BK;
  const size_t K = (size_t)p.K;
  const uint8_t* A = (const uint8_t*)p.A;
  const uint8_t* Be = (const uint8_t*)p.B + (size_t)e * N * K;
  const float* a_scales = (const float*)p.a_scales;
  const float* b_scales = (const float*)p.b_scales;

  LoadPlan lp;
  const int lrow = lane >> 3, slot = lane & 7;
#pragma unroll
  for (int i = 0; i < 2; i++) {                                // wave w: A rows [16w, 16w+16)
    const int r = wave * 16 + i * 8 + lrow;
    const int gr = row0 + min(r, rows - 1);                    // ragged tail: reuse a valid row
    lp.a_src[i] = A + (size_t)gr * K + (size_t)((slot ^ swz8(r)) * 16);
    lp.a_dst[i] = (wave * 16 + i * 8) * BK;
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {                                // wave w: B rows [32w, 32w+32)
    const int r = wave * 32 + i * 8 + lrow;
    const int gn = min(n0 + r, N - 1);                         // N tail: reuse a valid row
    lp.b_src[i] = Be + (size_t)gn * K + (size_t)((slot ^ swz8(r)) * 16);
    lp.b_dst[i] = A_BYTES + (wave * 32 + i * 8) * BK;
  }
  if (lane < 16) {
    lp.ss_src = a_scales + (size_t)(row0 + min(wave * 16 + lane, rows - 1)) * KB;
  } else {                                                     // wave 0, lanes 16 and 17
    const int nb = min(n0 / 128 + (lane - 16), N / 128 - 1);
    lp.ss_src = b_scales + ((size_t)e * (N / 128) + nb) * KB;
  }
  lp.ss_dst = SS_OFF + wave * 32 * 4;
  lp.ss_lane = lane < 16 || (wave == 0 && lane < 18);

  FragPlan fp;
  const int wm = wave & 1, wn = wave >> 1;                     // wave tile: rows 64wm, cols 64wn
  const int fr = lane & 31, kq = lane >> 5;
#pragma unroll
  for (int f = 0; f < 2; f++) {
#pragma unroll
    for (int kh = 0; kh < 2; kh++)
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int c = kh * 4 + kq * 2 + j;                     // 16-byte K chunk of this lane
        const int ra = wm * 64 + f * 32 + fr;
        const int rb = wn * 64 + f * 32 + fr;
        fp.a_off[f][kh][j] = ra * BK + ((c ^ swz8(ra)) * 16);
        fp.b_off[f][kh][j] = A_BYTES + rb * BK + ((c ^ swz8(rb)) * 16);
      }
    const int ra = wm * 64 + f * 32 + fr;
    fp.as_off[f] = SS_OFF + (ra >> 4) * 128 + (ra & 15) * 4;
  }
  fp.bs_off = BS_OFF + (wn >> 1) * 4;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = (v16f){};

  // prologue: K blocks 0 and 1 in flight
  issue_stage(smem, lp, 0);
  if (KB > 1) issue_stage(smem + STAGE_BYTES, lp, 1);
  for (int kb = 0; kb < KB; kb++) {
    const int s = kb % STAGES, s2 = (kb + 2) % STAGES;
    if (kb + 1 < KB) wait_vmcnt<LOADS_PER_STAGE>(); else wait_vmcnt<0>();
    barrier();                                                 // stage s landed; stage s2 free
    bw_step(smem + s * STAGE_BYTES, smem + s2 * STAGE_BYTES, lp, fp, kb + 2 < KB, kb + 2, acc);
  }

  // ---- epilogue: lane holds row (fr) and columns 8g + 4kq + {0..3} of each fragment ----
#pragma unroll
  for (int mi = 0; mi < 2; mi++) {
    const int mloc = wm * 64 + mi * 32 + fr;
    if (mloc >= rows) continue;
    const size_t crow = (size_t)(row0 + mloc) * N;
#pragma unroll
    for (int ni = 0; ni < 2; ni++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int col = n0 + wn * 64 + ni * 32 + g * 8 + kq * 4;
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
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(NTHREADS);
  switch (out) {
    case kOutF32: hipLaunchKernelGGL(bw_fp8_grouped_kernel<kOutF32>, grid, block, 0, stream, a, n_blocks); break;
    case kOutBF16: hipLaunchKernelGGL(bw_fp8_grouped_kernel<kOutBF16>, grid, block, 0, stream, a, n_blocks); break;
    case kOutF16: hipLaunchKernelGGL(bw_fp8_grouped_kernel<kOutF16>, grid, block, 0, stream, a, n_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsg
