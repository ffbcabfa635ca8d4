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
// the other kernels), 4 waves (one per SIMD) of 128 x 128 as 8 x 8 fragments of 16 x 16, fp32
// accumulators in AGPRs. The conversions are VALU work in proportion to the wave tile's rows plus
// columns, and they, not the matrix unit, bound this kernel: 128 x 128 needs a third fewer per
// product than 64 x 128 (8 waves, two per SIMD measured 0.50 of the f16 peak). A 2-stage LDS ring of
// 256-K stages filled by buffer -> LDS copies (stage b+1 is copied while stage b is computed, one
// copy per step), one barrier per stage. A stage row is 128 bytes of codes and 16 bytes of scales.
// The MFMA is written by hand (see mfma_acc), so this file keeps that instruction's hazards itself.
//
// K order inside a stage. The sum over K does not depend on which K elements a lane feeds to
// which instruction, as long as both operands use the same assignment. Lane (r16, q) of a
// fragment takes bytes [32 q, 32 q + 32) of its row: for half h (0, 1) the 16-byte chunk 2 q + h,
// and for step s (0..3) of that half its dword s, i.e. K elements [64 q + 32 h + 8 s, + 8). Those
// 8 elements share the scale of 16-block 4 q + 2 h + s / 2, and the lane's four scale blocks are
// the dword q of the row's 16 scale bytes.
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
constexpr int NWAVES = 4, NTHREADS = NWAVES * kWave;
constexpr int WM = 128, WN = 128;                  // wave tile (one wave per SIMD)
constexpr int MI = WM / 16, NJ = WN / 16;          // 8 x 8 fragments of 16 x 16
constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;        // 32 KiB each
constexpr int SA_BYTES = BM * SROWB, SB_BYTES = BN * SROWB;    // 4 KiB each
constexpr int A_OFF = 0, B_OFF = A_BYTES, SA_OFF = B_OFF + B_BYTES, SB_OFF = SA_OFF + SA_BYTES;
constexpr int STAGE_BYTES = SB_OFF + SB_BYTES;                  // 72 KiB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;                      // 144 KiB of 160
constexpr int D_INSTR = A_BYTES / 1024 / NWAVES;                // 8 copies of 1 KiB per operand
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(SA_BYTES == 4 * 1024 && NWAVES == 4, "scale copies: 1 KiB of A and of B per wave");

struct NvLoadPlan {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc, sa_rsrc, sb_rsrc;
  uint32_t voff[D_INSTR];  // data copies: per-lane offset of copy i (rows and swizzled chunk)
  uint32_t s_voff;         // scale copies: this lane's row
  int d_dst, s_dst;        // LDS destinations inside a stage's A / B and scale regions
};

// Copy c (of COPIES per wave) of stage kb into the stage at `st`: 8 KiB of A codes, 8 KiB of B
// codes and 1 KiB each of A and B scales per wave.
constexpr int COPIES = 2 * D_INSTR + 2;
__device__ __forceinline__ void copy_one(uint8_t* __restrict__ st, const NvLoadPlan& lp, int kb, int c) {
  const uint32_t k = (uint32_t)__builtin_amdgcn_readfirstlane(kb);
  if (c < D_INSTR)
    buf2lds16(lp.a_rsrc, lp.voff[c], k * ROWB, as_lds(st + A_OFF + lp.d_dst + c * 1024));
  else if (c < 2 * D_INSTR)
    buf2lds16(lp.b_rsrc, lp.voff[c - D_INSTR], k * ROWB, as_lds(st + B_OFF + lp.d_dst + (c - D_INSTR) * 1024));
  else if (c == 2 * D_INSTR)
    buf2lds16(lp.sa_rsrc, lp.s_voff, k * SROWB, as_lds(st + SA_OFF + lp.s_dst));
  else
    buf2lds16(lp.sb_rsrc, lp.s_voff, k * SROWB, as_lds(st + SB_OFF + lp.s_dst));
}
__device__ __forceinline__ void copy_stage(uint8_t* __restrict__ st, const NvLoadPlan& lp, int kb) {
#pragma unroll
  for (int c = 0; c < COPIES; c++) copy_one(st, lp, kb, c);
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

// Two e2m1 codes (byte `sel` of d) to f16, exactly (scale input 1).
__device__ __forceinline__ h2 cvt_fp4_pair(uint32_t d, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
  }
}

// acc += b^T-fragment x a-fragment, in place. Written as an instruction with the accumulator
// tied to its AGPRs: through the builtin the register allocator gives the result new AGPRs and
// copies, which with all 256 AGPRs holding accumulators spills into VGPRs.
// The compiler does not see this instruction's hazards, so the code around it keeps them:
//  * a VALU write of a source VGPR needs 2 wait states before the MFMA reads it (the compiler's
//    own MFMA hazard rules ask for that many after a VALU write of a source). The operands of
//    a step are built during the previous step, but the compiler may place their last writes (or
//    register moves) right at the step boundary, so the first MFMA of every step (WAIT = true)
//    starts with s_nop 4 (5 wait states, a margin over the 2 required); the others follow it by
//    at least one instruction more than it.
//  * the sources stay live until the end of the step (keep_live), so no VALU overwrites them
//    while the step's MFMAs read them; the accumulators are never VALU-written in the K loop.
//  * VALU reads of the results wait explicitly before the epilogue, and the accumulators are
//    zeroed well before the first MFMA.
template <bool WAIT>
__device__ __forceinline__ void mfma_acc(v4f& acc, const h8& b, const h8& a) {
  if constexpr (WAIT)
    asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
  else
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// An empty use that keeps a value in its registers up to this point.
__device__ __forceinline__ void keep_live(const h8& x) { asm volatile("" ::"v"(x)); }

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
  const int wm = wave >> 1, wn = wave & 1;                        // rows 128 wm, cols 128 wn
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
    lp.sa_rsrc = make_rsrc((const uint8_t*)p.a_scales + (size_t)row0 * srow, (uint64_t)rows * srow);
    lp.sb_rsrc = make_rsrc((const uint8_t*)p.b_scales + ((size_t)e * N + n0) * srow, (uint64_t)ncols * srow);
    {
      const int lrow = lane >> 3, slot = lane & 7;
      // copy i of wave w covers rows 64 w + 8 i + lrow; swz8 of such a row is lrow ^ (i & 1)
#pragma unroll
      for (int i = 0; i < D_INSTR; i++)
        lp.voff[i] = (uint32_t)((wave * 64 + i * 8 + lrow) * rowb + ((slot ^ lrow ^ (i & 1)) * 16));
      lp.d_dst = wave * D_INSTR * 1024;
      // scale copies of wave w: rows 64 w + lane of A and of B, 16 bytes each, row after row
      lp.s_voff = (uint32_t)((wave * 64 + lane) * srow);
      lp.s_dst = wave * 1024;
    }

    v4f acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
        asm volatile("" : "+a"(acc[i][j]));   // written to its AGPRs here, before the wait below
      }
    // wait states between those VALU writes and the first MFMA that reads them
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

    copy_stage(smem, lp, 0);
    wait_vmcnt<0>();
    barrier();

    for (int b = 0; b < KB; b++) {
      const uint8_t* st = smem + (b & 1) * STAGE_BYTES;
      // stage b+1 goes into the other buffer, whose last reads (stage b-1) ended before the
      // barrier that closed stage b-1; its copies are spread one per step over steps 1..18, so
      // that no run of copies holds up this wave's MFMA issue (in the last stage they repeat
      // stage KB-1 into a buffer that is not read again: a branch around them would stop the
      // step loop from being unrolled, which this kernel requires)
      uint8_t* const nxt = smem + ((b + 1) & 1) * STAGE_BYTES;

      // Scales of the stage: lane's dword of each A and B fragment row, decoded per half h into
      // f16 pairs (the scale of steps 4h, 4h+1 in [0], of 4h+2, 4h+3 in [1]).
      h2 as2[MI][2], bs2[NJ][2];
#pragma unroll
      for (int i = 0; i < MI; i++) {
        const uint32_t sd = *(const uint32_t*)(st + sa_off + i * 16 * SROWB);
        as2[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sd, 1.0f, false);
        as2[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sd, 1.0f, true);
      }
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const uint32_t sd = *(const uint32_t*)(st + sb_off + j * 16 * SROWB);
        bs2[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sd, 1.0f, false);
        bs2[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sd, 1.0f, true);
      }
      // A codes: the lane's 16 bytes of each fragment row for steps 0-3 (half 0); those of half 1
      // replace them at step 3, once the conversions for steps 1-3 are done
      v4i apk[MI];
#pragma unroll
      for (int i = 0; i < MI; i++) apk[i] = lds_read16(st + da[0] + i * 16 * ROWB);

      // 64 steps k = 8 u + j: step u of the stage's K (dword u of every lane's 32 bytes) against
      // B fragment j. Each step issues its 8 MFMAs, then decodes the B operand of step k+1, reads
      // the B dword of step k+2 and converts A fragment j for step u+1, so the VALU work of one
      // step runs under the previous step's MFMAs.
      auto b_dword = [&](int k) {
        const int u = k >> 3, j = k & 7;
        return *(const uint32_t*)(st + db[u >> 2] + j * 16 * ROWB + 4 * (u & 3));
      };
      auto scale_of = [](const h2 (&pr)[2], int u) {
        const h2 p2 = pr[u >> 2];
        return (u & 2) ? (h2){p2[1], p2[1]} : (h2){p2[0], p2[0]};
      };
      h8 avc[MI], avn[MI];
#pragma unroll
      for (int i = 0; i < MI; i++) avc[i] = decode8((uint32_t)apk[i][0], scale_of(as2[i], 0));
      h8 bv = decode8(b_dword(0), scale_of(bs2[0], 0));
      uint32_t bw1 = b_dword(1);
      // Fully unrolled (the build fails otherwise): the hand-written MFMAs need every
      // accumulator in fixed AGPRs; indexed at run time they would move through VGPRs next to
      // instructions whose wait states the compiler does not know.
#pragma clang loop unroll(full)
      for (int k = 0; k < 64; k++) {
        const int u = k >> 3, j = k & 7;
        const int u1 = (k + 1) >> 3, j1 = (k + 1) & 7;
        uint32_t bw2 = 0;
        if (k + 2 < 64) bw2 = b_dword(k + 2);
        if (k == 24) {
#pragma unroll
          for (int i = 0; i < MI; i++) apk[i] = lds_read16(st + da[1] + i * 16 * ROWB);
        }
        const h2 sbn = scale_of(bs2[j1 & 7], u1 & 7);
        const h2 san = scale_of(as2[j], (u + 1) & 7);
        const uint32_t aw = (uint32_t)apk[j][(u + 1) & 3];
        h2 bn[4], an[4];
        // MFMA i, then two VALU ops: conversions of the B operand of step k+1 under MFMAs 0-1 and
        // their scaling under MFMAs 2-3; the same for A fragment j of step u+1 under MFMAs 4-7.
        // A product is scaled two MFMAs after its conversion, so no op waits on the one before.
#pragma unroll
        for (int i = 0; i < MI; i++) {
          __builtin_amdgcn_sched_barrier(0);
          if (i == 0)
            mfma_acc<true>(acc[i][j], bv, avc[i]);
          else
            mfma_acc<false>(acc[i][j], bv, avc[i]);
          const int p0 = 2 * (i & 1);
          if (i < 4) {
            if (k + 1 < 64) {
              if (i < 2) {
                bn[p0] = cvt_fp4_pair(bw1, p0);
                bn[p0 + 1] = cvt_fp4_pair(bw1, p0 + 1);
              } else {
                bn[p0] = bn[p0] * sbn;
                bn[p0 + 1] = bn[p0 + 1] * sbn;
              }
            }
          } else if (u < 7) {
            if (i < 6) {
              an[p0] = cvt_fp4_pair(aw, p0);
              an[p0 + 1] = cvt_fp4_pair(aw, p0 + 1);
            } else {
              an[p0] = an[p0] * san;
              an[p0 + 1] = an[p0 + 1] * san;
            }
          }
        }
        if (k >= 1 && k <= COPIES) copy_one(nxt, lp, min(b + 1, KB - 1), k - 1);
        __builtin_amdgcn_sched_barrier(0);
        // the operands read by this step's MFMAs stay live until here, so the registers written
        // above are others
        keep_live(bv);
        if (k + 1 < 64) bv = (h8){bn[0][0], bn[0][1], bn[1][0], bn[1][1], bn[2][0], bn[2][1], bn[3][0], bn[3][1]};
        if (u < 7) avn[j] = (h8){an[0][0], an[0][1], an[1][0], an[1][1], an[2][0], an[2][1], an[3][0], an[3][1]};
        if (j == NJ - 1) {
#pragma unroll
          for (int i = 0; i < MI; i++) {
            keep_live(avc[i]);
            avc[i] = avn[i];
          }
        }
        bw1 = bw2;
      }
      // this wave's copies of stage b+1 have landed and its reads of stage b are done; after the
      // barrier every wave's are
      wait_vmcnt<0>();
      barrier();
    }

    // the last MFMAs' results are read by VALU below: give them the wait states the compiler
    // cannot see through the instructions written by hand
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // epilogue: lane holds row r16 of each M fragment and columns 4 q .. 4 q + 3 of each N
    // fragment; one M fragment at a time, so that only its 32 accumulators sit in VGPRs
#pragma unroll
    for (int i = 0; i < MI; i++) {
      __builtin_amdgcn_sched_barrier(0);
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
