// MX block-scaled GEMM for gfx950 (MI355X): e4m3 / e2m1 elements, one e8m0 scale per 32
// K-elements per row of A and per row of B (the MX variant of the Triton Gluon page
// "Overlapping Accumulator Block-Scaled Matrix Multiplication": scales applied inside the
// matrix instruction, as its async_mma_scaled_impl does with tcgen05_mma_scaled; reference
// result A_ref @ B_ref^T of its make_problem).
//
// CDNA4 mapping: v_mfma_scale_f32_16x16x128_f8f6f4 takes one e8m0 scale per lane, so the scales
// are applied by the matrix unit, the fp32 accumulator chains through the instruction and no
// software promotion is needed. Block structure as in the blockwise kernel: 256 x 256 block
// tiles (super-tiles of two 128-row M-tiles of one expert), 8 waves of 64 x 128 as 4 x 8
// fragments of 16 x 16, A fragments resident and B fragments streamed two ahead, a 2-stage LDS
// ring filled by buffer -> LDS copies, one barrier per K block. The scales of a super-tile's
// rows are staged 8 K blocks at a time (one dword of four scales per row and K block).
//
// Lane layout of one 128-wide K block (probed on gfx950): the scale of (row r, 32-K chunk c) is
// supplied by lane 16 c + r, so lane (r16 = l % 16, q = l / 16) supplies chunk q of its row.
// e2m1: lane (r16, q) holds chunk q itself (16 bytes, low nibble = even K). e4m3: lane (r16, q)
// holds K [16 q, 16 q + 16) in bytes 0..15 and K [64 + 16 q, 64 + 16 q + 16) in bytes 16..31.
#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128, TILE_M = 128;
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int WM = 64, WN = 128;                  // wave tile
constexpr int MI = WM / 16, NJ = WN / 16;         // 4 x 8 fragments of 16 x 16
constexpr int STAGES = 2;
constexpr int SC_CHUNK = 8;                       // K blocks per staged scale chunk
constexpr int SC_BYTES = BM * SC_CHUNK * 4;       // 8 KiB per operand and chunk
constexpr int SC_INSTR = SC_BYTES / 256 / NWAVES; // 4 (4-byte copies, 64 lanes)

// element format codes of the f8f6f4 instruction: 0 = e4m3, 4 = e2m1
template <int F> struct Elem;
template <> struct Elem<1> { static constexpr int kRowBytes = 128; static constexpr int kCode = 0; };
template <> struct Elem<2> { static constexpr int kRowBytes = 64; static constexpr int kCode = 4; };

// KS: 128-K sub-blocks per stage of the LDS ring (2 for e2m1 x e2m1, so that a stage holds as
// many bytes and MFMA work as an e4m3 one). RA / RB: bytes of one tile row in a stage.
template <int FA, int FB, int KS>
struct Layout {
  static constexpr int RA = Elem<FA>::kRowBytes * KS, RB = Elem<FB>::kRowBytes * KS;
  static constexpr int A_BYTES = BM * RA, B_BYTES = BN * RB;       // per stage
  static constexpr int A_REGION = 0;
  static constexpr int B_REGION = STAGES * A_BYTES;
  static constexpr int SA_REGION = B_REGION + STAGES * B_BYTES;    // 2 chunks of A scales
  static constexpr int SB_REGION = SA_REGION + 2 * SC_BYTES;       // 2 chunks of B scales
  static constexpr int LDS_BYTES = SB_REGION + 2 * SC_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024 / NWAVES;          // 1 KiB copies per wave
  static constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;
  static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small for the copy split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// 16-byte chunk swizzle of a tile row: 128-byte rows (e4m3) use swz8; for 64-byte rows (e2m1)
// two rows share a 128-byte bank line, and rows of one parity take the four slot permutations.
template <int ROWB>
__device__ __forceinline__ int swzr(int r) {
  if constexpr (ROWB == 128) return swz8(r); else return (r >> 1) & 3;
}

template <int ROWB>
struct FragBase {
  int off[2];   // byte offsets (inside a tile, row r16 of fragment 0) of the lane's two chunks
};

// Lane (r16, q) offsets inside a tile: e4m3 chunks q and 4 + q of the 128-byte row, e2m1 chunk q
// of the 64-byte row. The swizzle of row 16 f + r16 depends on r16 only.
template <int ROWB>
__device__ __forceinline__ FragBase<ROWB> frag_base(int row, int r16, int q) {
  FragBase<ROWB> b;
  const int sw = swzr<ROWB>(r16);
  if constexpr (ROWB == 128) {
    b.off[0] = row * ROWB + ((q ^ sw) * 16);
    b.off[1] = row * ROWB + (((4 + q) ^ sw) * 16);
  } else {
    b.off[0] = row * ROWB + ((q ^ sw) * 16);
    b.off[1] = b.off[0];
  }
  return b;
}

template <int ROWB>
__device__ __forceinline__ v8i read_frag(const uint8_t* p, const FragBase<ROWB>& b) {
  if constexpr (ROWB == 128) {
    return cat(lds_read16(p + b.off[0]), lds_read16(p + b.off[1]));
  } else {
    const v4i v = lds_read16(p + b.off[0]);
    return (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
  }
}

template <int FA, int FB, int KS>
struct MxLoadPlan {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc, sa_rsrc, sb_rsrc;
  uint32_t a_voff[Layout<FA, FB, KS>::A_INSTR], b_voff[Layout<FA, FB, KS>::B_INSTR];
  uint32_t sc_voff_a;              // A scale chunk: lane part (row and dword inside the chunk)
  uint32_t sc_row8_a;              // A scale chunk: bytes of 8 rows of the scale tensor
  uint32_t sc_voff_b[SC_INSTR];    // B scale chunk: per copy (B rows are permuted, see b_col)
  int a_dst, b_dst;
};

// Copy i (of A_INSTR / B_INSTR per wave) of K block kb into the A or B half of a stage.
template <int FA, int FB, int KS>
__device__ __forceinline__ void mx_copy_a(uint8_t* __restrict__ da, const MxLoadPlan<FA, FB, KS>& lp, int kb, int i) {
  using L = Layout<FA, FB, KS>;
  buf2lds16(lp.a_rsrc, lp.a_voff[i], (uint32_t)__builtin_amdgcn_readfirstlane(kb) * L::RA,
            as_lds(da + lp.a_dst + i * 1024));
}
template <int FA, int FB, int KS>
__device__ __forceinline__ void mx_copy_b(uint8_t* __restrict__ db, const MxLoadPlan<FA, FB, KS>& lp, int kb, int i) {
  using L = Layout<FA, FB, KS>;
  buf2lds16(lp.b_rsrc, lp.b_voff[i], (uint32_t)__builtin_amdgcn_readfirstlane(kb) * L::RB,
            as_lds(db + lp.b_dst + i * 1024));
}

// Scale chunk c (K blocks 8c .. 8c+7) of the super-tile's 256 A rows and 256 B rows into
// [row][8 dwords] layouts; wave w copies rows 32 w .. 32 w + 31 of each.
template <int FA, int FB, int KS>
__device__ __forceinline__ void mx_issue_scales(uint8_t* __restrict__ dsa, uint8_t* __restrict__ dsb,
                                                const MxLoadPlan<FA, FB, KS>& lp, int chunk, int wave) {
  const uint32_t col = (uint32_t)__builtin_amdgcn_readfirstlane(chunk) * SC_CHUNK * 4;
#pragma unroll
  for (int i = 0; i < SC_INSTR; i++) {
    buf2lds4(lp.sa_rsrc, lp.sc_voff_a + col + i * lp.sc_row8_a, 0, as_lds(dsa + (wave * SC_INSTR + i) * 256));
    buf2lds4(lp.sb_rsrc, lp.sc_voff_b[i] + col, 0, as_lds(dsb + (wave * SC_INSTR + i) * 256));
  }
}

template <int FA, int FB>
__device__ __forceinline__ v4f mma(const v8i& b, const v8i& a, const v4f& c, int sb, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, Elem<FB>::kCode, Elem<FA>::kCode,
                                                          0, sb, 0, sa);
}

// Operand of sub-block h of a fragment read as two 16-byte chunks: with two e2m1 sub-blocks per
// stage, chunk q holds sub-block 0 and chunk 4 + q sub-block 1 of the lane's 32-K slice (the
// instruction reads 4 registers of an e2m1 operand, so the unused half costs nothing).
template <int KS>
__device__ __forceinline__ v8i sub_op(const v8i& x, int h) {
  if constexpr (KS == 1) return x;
  else return h == 0 ? x : (v8i){x[4], x[5], x[6], x[7], 0, 0, 0, 0};
}

template <int FA, int FB, int OUT, int KS>
__global__ __launch_bounds__(NTHREADS, 1) void mx_kernel(GemmArgs p, int n_blocks) {
  using L = Layout<FA, FB, KS>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int num_super = (p.num_tiles + 1) / 2;
  int s, nb;
  if (!work_item(num_super, n_blocks, 8, s, nb)) return;
  const int n0 = nb * BN, N = p.N, KB = p.K / (BK * KS);          // stages
  const size_t rowA = (size_t)p.K * Elem<FA>::kRowBytes / BK;      // bytes per row
  const size_t rowB = (size_t)p.K * Elem<FB>::kRowBytes / BK;
  constexpr int SCS = SC_CHUNK / KS;                                // stages per scale chunk
  const size_t srow = (size_t)p.K / 32;                                            // scale bytes per row
  const int wm = wave >> 1, wn = wave & 1;                  // rows 64 wm, cols 128 wn
  const int r16 = lane & 15, q = lane >> 4;
  const int ncols = min(BN, N - n0);

  // the super-tile's passes, as in the blockwise kernel
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

  const FragBase<L::RA> fa = frag_base<L::RA>(wm * WM + r16, r16, q);
  const FragBase<L::RB> fb = frag_base<L::RB>(wn * WN + r16, r16, q);
  const int base_sa = L::SA_REGION + (wm * WM + r16) * SC_CHUNK * 4;
  const int base_sb = L::SB_REGION + (wn * WN + r16) * SC_CHUNK * 4;

  for (int ps = 0; ps < npass; ps++) {
    const int e = __builtin_amdgcn_readfirstlane(ps == 0 ? e0 : e1);
    const int row0 = __builtin_amdgcn_readfirstlane(ps == 0 ? r0 : r1);
    const int rows = __builtin_amdgcn_readfirstlane(ps == 0 ? n0rows : n1rows);

    // Copy plan. Every row offset is in the per-lane offset, which the resource bounds check:
    // rows past the pass or past N read as zero.
    MxLoadPlan<FA, FB, KS> lp;
    lp.a_rsrc = make_rsrc((const uint8_t*)p.A + (size_t)row0 * rowA, (uint64_t)rows * rowA);
    lp.b_rsrc = make_rsrc((const uint8_t*)p.B + ((size_t)e * N + n0) * rowB, (uint64_t)ncols * rowB);
    lp.sa_rsrc = make_rsrc((const uint8_t*)p.a_scales + (size_t)row0 * srow, (uint64_t)rows * srow);
    lp.sb_rsrc = make_rsrc((const uint8_t*)p.b_scales + ((size_t)e * N + n0) * srow, (uint64_t)ncols * srow);
    {
      constexpr int CA = L::RA / 16, CB = L::RB / 16;            // 16-byte chunks per tile row
      constexpr int PA = 1024 / L::RA, PB = 1024 / L::RB;        // tile rows per 1 KiB copy
#pragma unroll
      for (int i = 0; i < L::A_INSTR; i++) {
        const int r = (wave * L::A_INSTR + i) * PA + lane / CA, slot = lane % CA;
        lp.a_voff[i] = (uint32_t)(r * rowA + ((slot ^ swzr<L::RA>(r)) * 16));
      }
      // LDS row r of the B half holds B row (r & 128) | b_col(r & 127) (and so do the B scales),
      // so that the epilogue stores 16 bytes per lane; the swizzle follows the LDS row
#pragma unroll
      for (int i = 0; i < L::B_INSTR; i++) {
        const int r = (wave * L::B_INSTR + i) * PB + lane / CB, slot = lane % CB;
        lp.b_voff[i] = (uint32_t)(((r & 128) | b_col(r & 127)) * rowB + ((slot ^ swzr<L::RB>(r)) * 16));
      }
      lp.a_dst = wave * L::A_INSTR * 1024;
      lp.b_dst = wave * L::B_INSTR * 1024;
      const int lrow = lane >> 3, dw = lane & 7;                 // scale chunk: 8 rows x 8 dwords
      lp.sc_voff_a = (uint32_t)((wave * 32 + lrow) * srow + dw * 4);
      lp.sc_row8_a = (uint32_t)(8 * srow);
#pragma unroll
      for (int i = 0; i < SC_INSTR; i++) {
        const int r = wave * 32 + 8 * i + lrow;
        lp.sc_voff_b[i] = (uint32_t)(((r & 128) | b_col(r & 127)) * srow + dw * 4);
      }
    }

    v4f acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    // prologue: scale chunks 0 and 1, block 0 and the B half of block 1 (its A half goes out in
    // passes 0 and 1 of block 0, as in every block); block 0 published
    mx_issue_scales<FA, FB, KS>(smem + L::SA_REGION, smem + L::SB_REGION, lp, 0, wave);
    mx_issue_scales<FA, FB, KS>(smem + L::SA_REGION + SC_BYTES, smem + L::SB_REGION + SC_BYTES, lp, 1, wave);
#pragma unroll
    for (int i = 0; i < L::A_INSTR; i++) mx_copy_a<FA, FB, KS>(smem + L::A_REGION, lp, 0, i);
#pragma unroll
    for (int i = 0; i < L::B_INSTR; i++) mx_copy_b<FA, FB, KS>(smem + L::B_REGION, lp, 0, i);
#pragma unroll
    for (int i = 0; i < L::B_INSTR; i++) mx_copy_b<FA, FB, KS>(smem + L::B_REGION + L::B_BYTES, lp, min(1, KB - 1), i);
    wait_vmcnt<0>();
    barrier();

    // lane (r16, q) supplies the scale of chunk q: byte q of the row's dword, moved to byte 0
    // g: 128-K sub-block index (stage b holds sub-blocks KS b .. KS b + KS - 1)
    auto scale_a = [&](int g, int i) {
      const int so = ((g / SC_CHUNK) & 1) * SC_BYTES + (g % SC_CHUNK) * 4;
      return (int)(*(const uint32_t*)(smem + base_sa + so + i * 16 * SC_CHUNK * 4) >> (8 * q));
    };
    auto scale_b = [&](int g, int j) {
      const int so = ((g / SC_CHUNK) & 1) * SC_BYTES + (g % SC_CHUNK) * 4;
      return (int)(*(const uint32_t*)(smem + base_sb + so + j * 16 * SC_CHUNK * 4) >> (8 * q));
    };

    // A fragments and scales of the block stay in registers; B fragments and their scales
    // stream through 3-deep queues two fragments ahead
    v8i af[MI], bq[3];
    int sa[MI][KS], sbq[3][KS];
#pragma unroll
    for (int i = 0; i < MI; i++) {
      af[i] = read_frag<L::RA>(smem + L::A_REGION + i * 16 * L::RA, fa);
#pragma unroll
      for (int h = 0; h < KS; h++) sa[i][h] = scale_a(h, i);
    }
    bq[0] = read_frag<L::RB>(smem + L::B_REGION, fb);
    bq[1] = read_frag<L::RB>(smem + L::B_REGION + 16 * L::RB, fb);
#pragma unroll
    for (int h = 0; h < KS; h++) {
      sbq[0][h] = scale_b(h, 0);
      sbq[1][h] = scale_b(h, 1);
    }

    // copies per wave and pass: the A half of a block over passes 0 and 1, the B half over
    // passes 6 and 7, each after the second or fourth MFMA of the pass
    constexpr int A_PP = L::A_INSTR / 2, B_PP = L::B_INSTR / 2;
    static_assert(A_PP >= 1 && A_PP <= 2 && B_PP >= 1 && B_PP <= 2, "copy schedule");

    for (int b = 0; b < KB; b++) {
      const int S = b & 1;
      const int soa = S * L::A_BYTES, sob = S * L::B_BYTES;                 // this block's stage
      const int sna = (S ^ 1) * L::A_BYTES, snb = (S ^ 1) * L::B_BYTES;
      const int bn = min(b + 1, KB - 1);
      // passes 0..5: B fragment j against the 4 resident A fragments (with two sub-blocks per
      // stage: sub-block 0 for all four, then sub-block 1, so chained MFMAs are four apart), MFMAs
      // at raised wave priority; B fragment j + 2 is read in two halves (after the first and third MFMA) and
      // its scale after the third. Passes 0 and 1 also copy the A half of block b+1 into the
      // other stage (freed by the barrier of block b-1; its B half went out in passes 6 and 7
      // of block b-1). Each MFMA with what follows it is a scheduling region of its own.
#pragma unroll
      for (int j = 0; j < NJ - 2; j++) {
        __builtin_amdgcn_sched_barrier(0);
        v4i lo, hi;
        int sbn[KS];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h = 0; h < KS; h++)
#pragma unroll
        for (int i = 0; i < MI; i++) {
          acc[i][j] = mma<FA, FB>(sub_op<KS>(bq[j % 3], h), sub_op<KS>(af[i], h), acc[i][j], sbq[j % 3][h], sa[i][h]);
          if (h < KS - 1) {
            __builtin_amdgcn_sched_barrier(0);
            continue;
          }
          if (j < 2 && (i & 1) && (i >> 1) < A_PP)
            mx_copy_a<FA, FB, KS>(smem + L::A_REGION + sna, lp, bn, j * A_PP + (i >> 1));
          if (j + 2 < NJ && i == 0) lo = lds_read16(smem + L::B_REGION + sob + (j + 2) * 16 * L::RB + fb.off[0]);
          if (j + 2 < NJ && i == 2) {
            if constexpr (L::RB == 128) hi = lds_read16(smem + L::B_REGION + sob + (j + 2) * 16 * L::RB + fb.off[1]);
#pragma unroll
            for (int h = 0; h < KS; h++) sbn[h] = scale_b(KS * b + h, j + 2);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (j + 2 < NJ) {
          if constexpr (L::RB == 128) bq[(j + 2) % 3] = cat(lo, hi);
          else bq[(j + 2) % 3] = (v8i){lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
#pragma unroll
          for (int h = 0; h < KS; h++) sbq[(j + 2) % 3][h] = sbn[h];
        }
        // pin the previous pass's MFMAs (complete by now) ahead of this point, so that the
        // compiler does not sink them past the loop's branch
        if (j > 0) {
#pragma unroll
          for (int i = 0; i < MI; i++) asm volatile("" : "+v"(acc[i][j - 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage S fully read (its last read was in pass 5), block b+1 landed: publish it
      wait_vmcnt<0>();
      wait_lds_reads();
      barrier();
      // scales of chunk c+1 replace those of chunk c-1 while block 8c is computed
      if (b % SCS == 0 && b > 0) {
        const int cb = ((b / SCS + 1) & 1) * SC_BYTES;
        mx_issue_scales<FA, FB, KS>(smem + L::SA_REGION + cb, smem + L::SB_REGION + cb, lp, b / SCS + 1, wave);
      }
#pragma unroll
      for (int i = 0; i < MI; i++) asm volatile("" : "+v"(acc[i][NJ - 3]));
      __builtin_amdgcn_sched_barrier(0);
      // pass 6 with the first copies of the B half of block b+2 into stage S (past the last
      // block they repeat block KB-1 into a stage that is not read again)
#pragma unroll
      for (int h = 0; h < KS; h++)
#pragma unroll
      for (int i = 0; i < MI; i++) {
        acc[i][NJ - 2] = mma<FA, FB>(sub_op<KS>(bq[(NJ - 2) % 3], h), sub_op<KS>(af[i], h), acc[i][NJ - 2],
                                     sbq[(NJ - 2) % 3][h], sa[i][h]);
        if ((i & 1) && (i >> 1) < B_PP && h == KS - 1)
          mx_copy_b<FA, FB, KS>(smem + L::B_REGION + sob, lp, min(b + 2, KB - 1), i >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // pass 7: last B fragment; each A fragment and its scale are refilled from block b+1
      // right after their MFMA; the rest of the B half of block b+2; then the first two B
      // fragments of block b+1 and their scales are read
#pragma unroll
      for (int h = 0; h < KS; h++)
#pragma unroll
      for (int i = 0; i < MI; i++) {
        acc[i][NJ - 1] = mma<FA, FB>(sub_op<KS>(bq[(NJ - 1) % 3], h), sub_op<KS>(af[i], h), acc[i][NJ - 1],
                                     sbq[(NJ - 1) % 3][h], sa[i][h]);
        if (h < KS - 1) {
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        af[i] = read_frag<L::RA>(smem + L::A_REGION + sna + i * 16 * L::RA, fa);
#pragma unroll
        for (int h = 0; h < KS; h++) sa[i][h] = scale_a(KS * bn + h, i);
        if ((i & 1) && (i >> 1) < B_PP)
          mx_copy_b<FA, FB, KS>(smem + L::B_REGION + sob, lp, min(b + 2, KB - 1), B_PP + (i >> 1));
        __builtin_amdgcn_sched_barrier(0);
      }
      bq[0] = read_frag<L::RB>(smem + L::B_REGION + snb, fb);
      bq[1] = read_frag<L::RB>(smem + L::B_REGION + snb + 16 * L::RB, fb);
#pragma unroll
      for (int h = 0; h < KS; h++) {
        sbq[0][h] = scale_b(KS * bn + h, 0);
        sbq[1][h] = scale_b(KS * bn + h, 1);
      }
#pragma unroll
      for (int i = 0; i < MI; i++) asm volatile("" : "+v"(acc[i][NJ - 2]));
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();

    // epilogue: lane holds row r16 of each M fragment and, over N fragments 2 jj and 2 jj + 1,
    // columns 32 jj + 8 q .. 32 jj + 8 q + 7 of its 128-column block (see b_col)
#pragma unroll
    for (int i = 0; i < MI; i++) {
      const int mloc = wm * WM + i * 16 + r16;
      if (mloc >= rows) continue;
      const size_t crow = (size_t)(row0 + mloc) * N;
#pragma unroll
      for (int jj = 0; jj < NJ / 2; jj++) {
        const int col = n0 + wn * WN + jj * 32 + q * 8;
        if (col < N) store8<OUT>(p.C, crow + col, acc[i][2 * jj], acc[i][2 * jj + 1]);
      }
    }
    if (ps + 1 < npass) barrier();   // every wave is past its last LDS read before the next pass
  }
}

template <int FA, int FB, int KS = 1>
hipError_t launch_fmt(const GemmArgs& a, int out, hipStream_t stream, dim3 grid, int n_blocks) {
  dim3 block(NTHREADS);
  switch (out) {
    case kOutF32: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutF32, KS>), grid, block, 0, stream, a, n_blocks); break;
    case kOutBF16: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutBF16, KS>), grid, block, 0, stream, a, n_blocks); break;
    case kOutF16: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutF16, KS>), grid, block, 0, stream, a, n_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx(const GemmArgs& a, int fmt_a, int fmt_b, int out, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long blocks = (long long)((a.num_tiles + 1) / 2) * n_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0LL) return hipErrorInvalidValue;
  const dim3 grid(grid_for(blocks));
  if (fmt_a == 1 && fmt_b == 1) return launch_fmt<1, 1>(a, out, stream, grid, n_blocks);
  if (fmt_a == 1 && fmt_b == 2) return launch_fmt<1, 2>(a, out, stream, grid, n_blocks);
  if (fmt_a == 2 && fmt_b == 1) return launch_fmt<2, 1>(a, out, stream, grid, n_blocks);
  if (fmt_a == 2 && fmt_b == 2) {
    // 256-K stages when K is a multiple of 256
    if ((a.K / BK) % 2 == 0) return launch_fmt<2, 2, 2>(a, out, stream, grid, n_blocks);
    return launch_fmt<2, 2, 1>(a, out, stream, grid, n_blocks);
  }
  return hipErrorInvalidValue;
}

}  // namespace bsg
