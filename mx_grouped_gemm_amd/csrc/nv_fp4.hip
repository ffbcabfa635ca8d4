// nvfp4 block-scaled GEMM for gfx950 (MI355X): e2m1 elements with one e4m3fn scale per 16
// K-elements per row of A and per row of B (the nvfp4 format of the Triton Gluon page
// "Overlapping Accumulator Block-Scaled Matrix Multiplication", random_quantized_tensor with
// VEC_SIZE 16; reference result A_ref @ B_ref^T of its make_problem).
//
// CDNA4 mapping. The gfx950 scaled matrix instruction takes one power-of-two (e8m0) scale per
// 32 K-elements, so it cannot apply an e4m3 scale per 16. Each lane instead folds the scale into
// its operand: v_cvt_scalef32_pk_f16_fp4 turns two e2m1 codes into f16 exactly (its scale input
// applies only the exponent, so it is fed 1.0), and v_pk_mul_f16 multiplies the pair by the e4m3
// scale, also decoded to f16. Both steps are exact: an e2m1 value times an e4m3 scale has at most
// 6 significant bits and lies in [2^-10, 2688], inside f16's normal range. The products then run
// through v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//
// Block structure: 256 x 256 block tiles (super-tiles of two 128-row M-tiles of one expert, as in
// the other kernels), 8 waves of 64 x 128 as 4 x 8 fragments of 16 x 16, a 2-stage LDS ring of
// 256-K stages filled by buffer -> LDS copies (stage b+1 is copied while stage b is computed),
// one barrier per stage. A stage row is 128 bytes of codes and 16 bytes of scales.
//
// K order inside a stage. The sum over K does not depend on which K elements a lane feeds to
// which instruction, as long as both operands use the same assignment. Lane (r16, q) of a
// fragment takes bytes [32 q, 32 q + 32) of its row: for half h (0, 1) the 16-byte chunk 2 q + h,
// and for step s (0..3) of that half its dword s, i.e. K elements [64 q + 32 h + 8 s, + 8). Those
// 8 elements share the scale of 16-block 4 q + 2 h + s / 2, and the lane's four scale blocks are
// the dword q of the row's 16 scale bytes.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, TILE_M = 128;
constexpr int KSTAGE = 256;                        // K elements per stage
constexpr int ROWB = KSTAGE / 2;                   // 128 bytes of e2m1 codes per row and stage
constexpr int SROWB = KSTAGE / 16;                 // 16 scale bytes per row and stage
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int WM = 64, WN = 128;                   // wave tile
constexpr int MI = WM / 16, NJ = WN / 16;          // 4 x 8 fragments of 16 x 16
constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;        // 32 KiB each
constexpr int SA_BYTES = BM * SROWB, SB_BYTES = BN * SROWB;    // 4 KiB each
constexpr int A_OFF = 0, B_OFF = A_BYTES, SA_OFF = B_OFF + B_BYTES, SB_OFF = SA_OFF + SA_BYTES;
constexpr int STAGE_BYTES = SB_OFF + SB_BYTES;                  // 72 KiB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;                      // 144 KiB of 160
constexpr int D_INSTR = A_BYTES / 1024 / NWAVES;                // 4 copies of 1 KiB per operand
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(SA_BYTES == 4 * 1024 && NWAVES == 8, "scale copies: one 1 KiB copy per wave");

struct NvLoadPlan {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc, s_rsrc;  // s_rsrc: A scales (waves 0-3) or B (4-7)
  uint32_t voff[D_INSTR];  // data copies: per-lane offset of copy i (rows and swizzled chunk)
  uint32_t s_voff;         // scale copy: this lane's row
  int d_dst, s_dst;        // LDS destinations inside a stage
};

// Copies of stage kb into the stage at `st`: 4 KiB of A codes, 4 KiB of B codes and 1 KiB of
// scales per wave.
__device__ __forceinline__ void copy_stage(uint8_t* __restrict__ st, const NvLoadPlan& lp, int kb) {
  const uint32_t k = (uint32_t)__builtin_amdgcn_readfirstlane(kb);
#pragma unroll
  for (int i = 0; i < D_INSTR; i++) {
    buf2lds16(lp.a_rsrc, lp.voff[i], k * ROWB, as_lds(st + A_OFF + lp.d_dst + i * 1024));
    buf2lds16(lp.b_rsrc, lp.voff[i], k * ROWB, as_lds(st + B_OFF + lp.d_dst + i * 1024));
  }
  buf2lds16(lp.s_rsrc, lp.s_voff, k * SROWB, as_lds(st + lp.s_dst));
}

// 8 f16 operand values from one dword of e2m1 codes (bytes 0..3, two codes each), times the
// scale `sc` (the same f16 in both halves).
__device__ __forceinline__ h8 decode8(uint32_t d, h2 sc) {
  const h2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sc;
  const h2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sc;
  const h2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sc;
  const h2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sc;
  return (h8){c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
}

// The two e4m3 scales of half h of a lane's scale dword (bytes 2h and 2h+1) as f16, each
// broadcast to both halves of a pair: [0] for steps 0-1, [1] for steps 2-3.
template <int H>
__device__ __forceinline__ void half_scales(uint32_t sd, h2 (&out)[2]) {
  const h2 p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sd, 1.0f, H != 0);
  out[0] = (h2){p[0], p[0]};
  out[1] = (h2){p[1], p[1]};
}

template <int OUT>
__global__ __launch_bounds__(NTHREADS, 1) void nv_fp4_kernel(GemmArgs p, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int num_super = (p.num_tiles + 1) / 2;
  int s, nb;
  if (!work_item(num_super, n_blocks, 8, s, nb)) return;
  const int n0 = nb * BN, N = p.N, KB = p.K / KSTAGE;
  const size_t rowb = (size_t)p.K / 2, srow = (size_t)p.K / 16;   // bytes per row: codes, scales
  const int wm = wave >> 1, wn = wave & 1;                        // rows 64 wm, cols 128 wn
  const int r16 = lane & 15, q = lane >> 4;
  const int ncols = min(BN, N - n0);

  // the super-tile's passes: one 256-row pass when its two M-tiles are consecutive rows of one
  // expert, else one pass per tile
  const TileRows t0 = tile_rows(p.expert_ids, p.tile_offsets, 2 * s, p.M, TILE_M, p.num_experts);
  TileRows t1 = {0, 0, 0};
  if (2 * s + 1 < p.num_tiles)
    t1 = tile_rows(p.expert_ids, p.tile_offsets, 2 * s + 1, p.M, TILE_M, p.num_experts);
  int e0 = t0.expert, r0 = t0.row0, n0rows = t0.rows, e1 = t1.expert, r1 = t1.row0, n1rows = t1.rows;
  int npass;
  if (t0.rows == TILE_M && t1.rows > 0 && t1.expert == t0.expert && t1.row0 == t0.row0 + TILE_M) {
    n0rows = TILE_M + t1.rows;
    npass = 1;
  } else if (t0.rows > 0) {
    npass = t1.rows > 0 ? 2 : 1;
  } else {
    e0 = e1; r0 = r1; n0rows = n1rows;
    npass = t1.rows > 0 ? 1 : 0;
  }

  // LDS read offsets inside a stage (row r16 of fragment 0): chunk 2 q + h of the 128-byte row,
  // swizzled; the swizzle of row 16 f + r16 depends on r16 only
  const int sw = swz8(r16);
  int da[2], db[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    da[h] = A_OFF + (wm * WM + r16) * ROWB + (((2 * q + h) ^ sw) * 16);
    db[h] = B_OFF + (wn * WN + r16) * ROWB + (((2 * q + h) ^ sw) * 16);
  }
  const int sa_off = SA_OFF + (wm * WM + r16) * SROWB + 4 * q;
  const int sb_off = SB_OFF + (wn * WN + r16) * SROWB + 4 * q;

  for (int ps = 0; ps < npass; ps++) {
    const int e = __builtin_amdgcn_readfirstlane(ps == 0 ? e0 : e1);
    const int row0 = __builtin_amdgcn_readfirstlane(ps == 0 ? r0 : r1);
    const int rows = __builtin_amdgcn_readfirstlane(ps == 0 ? n0rows : n1rows);

    // Copy plan. Every row offset sits in the per-lane offset, which the resource bounds check:
    // rows past the pass or past N read as zero (codes and scales).
    NvLoadPlan lp;
    lp.a_rsrc = make_rsrc((const uint8_t*)p.A + (size_t)row0 * rowb, (uint64_t)rows * rowb);
    lp.b_rsrc = make_rsrc((const uint8_t*)p.B + ((size_t)e * N + n0) * rowb, (uint64_t)ncols * rowb);
    if (wave < 4)
      lp.s_rsrc = make_rsrc((const uint8_t*)p.a_scales + (size_t)row0 * srow, (uint64_t)rows * srow);
    else
      lp.s_rsrc = make_rsrc((const uint8_t*)p.b_scales + ((size_t)e * N + n0) * srow, (uint64_t)ncols * srow);
    {
      const int lrow = lane >> 3, slot = lane & 7;
      // copy i of wave w covers rows 32 w + 8 i + lrow; swz8 of such a row is lrow ^ (i & 1)
#pragma unroll
      for (int i = 0; i < D_INSTR; i++)
        lp.voff[i] = (uint32_t)((wave * 32 + i * 8 + lrow) * rowb + ((slot ^ lrow ^ (i & 1)) * 16));
      lp.d_dst = wave * D_INSTR * 1024;
      // scale copy of wave w: rows 64 (w % 4) + lane, 16 bytes each, stored row after row
      lp.s_voff = (uint32_t)(((wave & 3) * 64 + lane) * srow);
      lp.s_dst = (wave < 4 ? SA_OFF : SB_OFF) + (wave & 3) * 1024;
    }

    v4f acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    copy_stage(smem, lp, 0);
    wait_vmcnt<0>();
    barrier();

    for (int b = 0; b < KB; b++) {
      const uint8_t* st = smem + (b & 1) * STAGE_BYTES;
      // stage b+1 goes into the other buffer, whose last reads (stage b-1) ended before the
      // barrier that closed stage b-1
      if (b + 1 < KB) copy_stage(smem + ((b + 1) & 1) * STAGE_BYTES, lp, b + 1);

      uint32_t asd[MI], bsd[NJ];
#pragma unroll
      for (int i = 0; i < MI; i++) asd[i] = *(const uint32_t*)(st + sa_off + i * 16 * SROWB);
#pragma unroll
      for (int j = 0; j < NJ; j++) bsd[j] = *(const uint32_t*)(st + sb_off + j * 16 * SROWB);

      auto half = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        v4i apk[MI], bpk[NJ];
#pragma unroll
        for (int i = 0; i < MI; i++) apk[i] = lds_read16(st + da[h] + i * 16 * ROWB);
#pragma unroll
        for (int j = 0; j < NJ; j++) bpk[j] = lds_read16(st + db[h] + j * 16 * ROWB);
        h2 asc[MI][2], bsc[NJ][2];
#pragma unroll
        for (int i = 0; i < MI; i++) half_scales<h>(asd[i], asc[i]);
#pragma unroll
        for (int j = 0; j < NJ; j++) half_scales<h>(bsd[j], bsc[j]);
#pragma unroll
        for (int t = 0; t < 4; t++) {
          h8 av[MI];
#pragma unroll
          for (int i = 0; i < MI; i++) av[i] = decode8((uint32_t)apk[i][t], asc[i][t >> 1]);
#pragma unroll
          for (int j = 0; j < NJ; j++) {
            const h8 bv = decode8((uint32_t)bpk[j][t], bsc[j][t >> 1]);
#pragma unroll
            for (int i = 0; i < MI; i++)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv, av[i], acc[i][j], 0, 0, 0);
          }
        }
      };
      half(std::integral_constant<int, 0>());
      half(std::integral_constant<int, 1>());
      // this wave's copies of stage b+1 have landed and its reads of stage b are done; after the
      // barrier every wave's are
      wait_vmcnt<0>();
      barrier();
    }

    // epilogue: lane holds row r16 of each M fragment and columns 4 q .. 4 q + 3 of each N fragment
#pragma unroll
    for (int i = 0; i < MI; i++) {
      const int mloc = wm * WM + i * 16 + r16;
      if (mloc >= rows) continue;
      const size_t crow = (size_t)(row0 + mloc) * N;
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const int col = n0 + wn * WN + j * 16 + q * 4;
        if (col < N) store4<OUT>(p.C, crow + col, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
    // no barrier needed before the next pass: the K loop ends with one, after the last reads
  }
}

}  // namespace

hipError_t launch_nvfp4(const GemmArgs& a, int out, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long blocks = (long long)((a.num_tiles + 1) / 2) * n_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0LL || a.K % KSTAGE) return hipErrorInvalidValue;
  const dim3 grid(grid_for(blocks)), block(NTHREADS);
  switch (out) {
    case kOutF32: hipLaunchKernelGGL(nv_fp4_kernel<kOutF32>, grid, block, 0, stream, a, n_blocks); break;
    case kOutBF16: hipLaunchKernelGGL(nv_fp4_kernel<kOutBF16>, grid, block, 0, stream, a, n_blocks); break;
    case kOutF16: hipLaunchKernelGGL(nv_fp4_kernel<kOutF16>, grid, block, 0, stream, a, n_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsg
