// MX block-scaled GEMM for gfx950 (MI355X): e4m3 / e2m1 elements, one e8m0 scale per 32
// K-elements per row of A and per row of B (the MX variant of the Triton Gluon page
// "Overlapping Accumulator Block-Scaled Matrix Multiplication": scales applied inside the
// matrix instruction, as its async_mma_scaled_impl does with tcgen05_mma_scaled; reference
// result A_ref @ B_ref^T of its make_problem).
//
// CDNA4 mapping: v_mfma_scale_f32_16x16x128_f8f6f4 takes one e8m0 scale per lane, so the scales
// are applied by the matrix unit, the fp32 accumulator chains through the instruction and no
// software promotion is needed. Block structure as in the blockwise kernel: a persistent grid
// (one workgroup per compute unit) over 256 x 256 work items (super-tiles of two 128-row M-tiles
// of one expert) with one copy pipeline across a workgroup's items, 8 waves of 64 x 128 as 4 x 8
// fragments of 16 x 16, A fragments resident and B fragments streamed two ahead, a 2-stage LDS
// ring filled by buffer -> LDS copies, one barrier per K block. The scales of a super-tile's
// rows are staged 8 K blocks at a time (one dword of four scales per row and K block).
//
// Lane layout of one 128-wide K block (probed on gfx950): the scale of (row r, 32-K chunk c) is
// supplied by lane 16 c + r, so lane (r16 = l % 16, q = l / 16) supplies chunk q of its row.
// e2m1: lane (r16, q) holds chunk q itself (16 bytes, low nibble = even K). e4m3: lane (r16, q)
// holds K [16 q, 16 q + 16) in bytes 0..15 and K [64 + 16 q, 64 + 16 q + 16) in bytes 16..31.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace bsg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
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
  static constexpr int B_REGION = 0;
  static constexpr int A_REGION = STAGES * B_BYTES;
  static constexpr int SA_REGION = A_REGION + STAGES * A_BYTES;    // 2 chunks of A scales
  static constexpr int SB_REGION = SA_REGION + 2 * SC_BYTES;       // 2 chunks of B scales
  static constexpr int LDS_BYTES = SB_REGION + 2 * SC_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024 / NWAVES;          // 1 KiB copies per wave
  static constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;
  static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small for the copy split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// 16-byte chunk swizzle of a tile row: chunk c of LDS row r sits at slot c ^ swzr(r). Banking of
// 16-byte reads, probed on gfx950 (timed reads of candidate layouts in isolation, and the LDS
// bank-conflict counter of this kernel): the LDS serves such a read 16 lanes at a time across
// 256 bytes of banks (64 x 4), and a group of 16 lanes holds every r16 once but is not 16
// consecutive lanes, so a layout is conflict-free only if the 16 lanes of each group land in 16
// different 16-byte slots of the 256 bytes. Each layout here was checked against every lane
// grouping that agrees with the probes and then measured: 0 conflict cycles for all three pairs.
// A lane reads chunk q (and 4 + q) of row r16 of a fragment. 128-byte rows: swzr, a bijection of
// r16 >> 1, with r16 & 1 spreads the rows (the slot is 8 (r16 & 1) + (c ^ swzr) modulo 16);
// 64-byte rows: (r16 >> 1) & 3 (the swizzle (r16 >> 2) & 3, conflict-free for a 32-lane,
// 512-byte service, left every read of the mixed pair's 64-byte rows two-way conflicted here).
template <int ROWB>
__device__ __forceinline__ int swzr(int r) {
  if constexpr (ROWB == 128) return (((r >> 2) & 3) << 1) | ((r >> 1) & 1);
  else return (r >> 1) & 3;
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
  uint32_t srow;                   // bytes of one row of the scale tensors
};

// LDS destinations are 32-bit LDS addresses: this wave's bases (see lds_bases) plus constants.
__device__ __forceinline__ lds_void* lds_ptr(uint32_t a) { return (lds_void*)(size_t)a; }

// This wave's copy destination bases: wa / wb for its part of an A / B tile, ws for its rows of a
// scale chunk. Re-derived through an empty asm at every stage so that the compiler forms each
// destination (base + constant) next to its copy instead of keeping every combination live in
// SGPRs.
struct LdsBases {
  uint32_t wa, wb, ws;
};
template <int FA, int FB, int KS>
__device__ __forceinline__ LdsBases lds_bases(const uint8_t* smem, int wave) {
  using L = Layout<FA, FB, KS>;
  const uint32_t s0 = (uint32_t)(size_t)as_lds(const_cast<uint8_t*>(smem));
  LdsBases l;
  l.wa = s0 + wave * L::A_INSTR * 1024;
  l.wb = s0 + wave * L::B_INSTR * 1024;
  l.ws = s0 + wave * SC_INSTR * 256;
  asm volatile("" : "+s"(l.wa), "+s"(l.wb), "+s"(l.ws));
  return l;
}

// Copy i (of A_INSTR / B_INSTR per wave) of K block kb to LDS address dst (the stage's A or B
// tile plus this wave's part).
template <int FA, int FB, int KS>
__device__ __forceinline__ void mx_copy_a(uint32_t dst, const MxLoadPlan<FA, FB, KS>& lp, int kb, int i) {
  using L = Layout<FA, FB, KS>;
  buf2lds16(lp.a_rsrc, lp.a_voff[i], (uint32_t)__builtin_amdgcn_readfirstlane(kb) * L::RA, lds_ptr(dst + i * 1024));
}
template <int FA, int FB, int KS>
__device__ __forceinline__ void mx_copy_b(uint32_t dst, const MxLoadPlan<FA, FB, KS>& lp, int kb, int i) {
  using L = Layout<FA, FB, KS>;
  buf2lds16(lp.b_rsrc, lp.b_voff[i], (uint32_t)__builtin_amdgcn_readfirstlane(kb) * L::RB, lds_ptr(dst + i * 1024));
}

// Scale chunk c (K blocks 8c .. 8c+7) of the super-tile's 256 A rows and 256 B rows, one dword
// (the four 32-K chunks of a K block) per row and K block. LDS row r of the B half holds B row
// (r & 128) | b_col(r & 127), as the B tile does. Two layouts:
// * by row (PK false): [row][8 dwords]; wave w copies rows 32 w .. 32 w + 31 of each
//   (instruction i: rows 32 w + 8 i + lane / 8, dword lane % 8). K block k of row r sits in dword
//   k ^ ((r >> 1) & 7): read by rows alone, the 16 rows of a fragment (32 bytes apart) stalled
//   the LDS for 6 cycles per read (2.7 times a conflict-free dword read, probed);
// * packed (PK true): the dwords a lane's fragments need side by side, so that one 16-byte read
//   gives a K block's dwords of 4 fragments. A: [64-row group][r16][K block slot][fragment f] for
//   row 64 g + 16 f + r16; B: [128-row group][r16][K block slot][fragment j] for LDS row
//   128 g + 16 j + r16. K block k of row group (g, r16) sits in slot k ^ ((r16 >> 1) & 7), and in
//   B rows of odd r16 the two 16-byte halves of a slot (fragments 0-3, 4-7) trade places, so that
//   the 16 rows that one read touches fall in 16 different bank slots (see swzr).
// The per-lane offsets are formed here, once per chunk (an empty asm keeps the compiler from
// keeping them live across the K loop).
template <int FA, int FB, int KS, bool PK>
__device__ __forceinline__ void mx_issue_scales(uint32_t dsa, uint32_t dsb, const MxLoadPlan<FA, FB, KS>& lp,
                                                int chunk, int wave) {
  const uint32_t col = (uint32_t)__builtin_amdgcn_readfirstlane(chunk) * SC_CHUNK * 4;
  int ln = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int i = 0; i < SC_INSTR; i++) {
    uint32_t va, vb;
    if constexpr (PK) {
      const int p = (wave * SC_INSTR + i) * 64 + ln;   // dword of the chunk this lane writes
      const int fa = p & 3, sa = (p >> 2) & 7, ra = (p >> 5) & 15, ga = p >> 9;
      va = (uint32_t)(ga * 64 + fa * 16 + ra) * lp.srow + (sa ^ ((ra >> 1) & 7)) * 4 + col;
      const int jb = p & 7, sb = (p >> 3) & 7, rb = (p >> 6) & 15, gb = p >> 10;
      const int lr = gb * 128 + (jb ^ ((rb & 1) << 2)) * 16 + rb;
      vb = (uint32_t)((lr & 128) | b_col(lr & 127)) * lp.srow + (sb ^ ((rb >> 1) & 7)) * 4 + col;
    } else {
      const int r = wave * 32 + 8 * i + (ln >> 3), dw = ln & 7;
      const int kd = dw ^ ((r >> 1) & 7);
      va = (uint32_t)r * lp.srow + kd * 4 + col;
      vb = (uint32_t)((r & 128) | b_col(r & 127)) * lp.srow + kd * 4 + col;
    }
    buf2lds4(lp.sa_rsrc, va, 0, lds_ptr(dsa + i * 256));
    buf2lds4(lp.sb_rsrc, vb, 0, lds_ptr(dsb + i * 256));
  }
}

// The scaled MFMA taking byte JS of sb and byte IS of sa as the lane's scales.
template <int FA, int FB, int JS, int IS>
__device__ __forceinline__ v4f mma_sel(const v8i& b, const v8i& a, const v4f& c, int sb, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, Elem<FB>::kCode, Elem<FA>::kCode,
                                                          JS, sb, IS, sa);
}
// jsel, isel in 0..3, constants once the pass loops are unrolled (the switch then folds away)
template <int FA, int FB>
__device__ __forceinline__ v4f mma_p(const v8i& b, const v8i& a, const v4f& c, int sb, int jsel, int sa, int isel) {
  switch (jsel * 4 + isel) {
    case 0: return mma_sel<FA, FB, 0, 0>(b, a, c, sb, sa);
    case 1: return mma_sel<FA, FB, 0, 1>(b, a, c, sb, sa);
    case 2: return mma_sel<FA, FB, 0, 2>(b, a, c, sb, sa);
    case 3: return mma_sel<FA, FB, 0, 3>(b, a, c, sb, sa);
    case 4: return mma_sel<FA, FB, 1, 0>(b, a, c, sb, sa);
    case 5: return mma_sel<FA, FB, 1, 1>(b, a, c, sb, sa);
    case 6: return mma_sel<FA, FB, 1, 2>(b, a, c, sb, sa);
    case 7: return mma_sel<FA, FB, 1, 3>(b, a, c, sb, sa);
    case 8: return mma_sel<FA, FB, 2, 0>(b, a, c, sb, sa);
    case 9: return mma_sel<FA, FB, 2, 1>(b, a, c, sb, sa);
    case 10: return mma_sel<FA, FB, 2, 2>(b, a, c, sb, sa);
    case 11: return mma_sel<FA, FB, 2, 3>(b, a, c, sb, sa);
    case 12: return mma_sel<FA, FB, 3, 0>(b, a, c, sb, sa);
    case 13: return mma_sel<FA, FB, 3, 1>(b, a, c, sb, sa);
    case 14: return mma_sel<FA, FB, 3, 2>(b, a, c, sb, sa);
    default: return mma_sel<FA, FB, 3, 3>(b, a, c, sb, sa);
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
__global__ __launch_bounds__(NTHREADS, 1) void mx_kernel(GemmArgs p, int n_blocks,
                                                        const int32_t* __restrict__ expert_ids,
                                                        const int32_t* __restrict__ tile_offsets,
                                                        void* __restrict__ C) {
  using L = Layout<FA, FB, KS>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::LDS_BYTES];
  const TileMap tm = {expert_ids, tile_offsets};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int items = ((p.num_tiles + 1) / 2) * n_blocks;
  const int N = p.N, KB = p.K / (BK * KS);                         // stages per unit
  const size_t rowA = (size_t)p.K * Elem<FA>::kRowBytes / BK;      // bytes per row
  const size_t rowB = (size_t)p.K * Elem<FB>::kRowBytes / BK;
  constexpr int SCS = SC_CHUNK / KS;                                // stages per scale chunk
  const int nchunks = (KB + SCS - 1) / SCS;                        // scale chunks per unit
  const size_t srow = (size_t)p.K / 32;                            // scale bytes per row
  const int wm = wave >> 1, wn = wave & 1;                  // rows 64 wm, cols 128 wn
  const int r16 = lane & 15, q = lane >> 4;
  // Consecutive stages of the units of this workgroup share one pipeline, as in the blockwise
  // kernel: the last two stages of a unit copy the first two of the next (and its first two scale
  // chunks), so only the first unit has a prologue and a unit's stores drain under the next one's
  // first passes. This needs an even number of stages per unit; with an odd number every unit
  // starts with its own prologue.
  const bool piped = (KB & 1) == 0;
  // Work order as in the blockwise kernel: the grid is a multiple of 8, block b runs on XCD b % 8,
  // and the blocks of one XCD take contiguous runs of logical items.
  const int xb = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;

  const FragBase<L::RA> fa = frag_base<L::RA>(wm * WM + r16, r16, q);
  const FragBase<L::RB> fb = frag_base<L::RB>(wn * WN + r16, r16, q);
  // Scale layout (see mx_issue_scales): packed for A and B of one format, by row for a mixed
  // pair. Measured at 8192^3 against reading each scale as a byte: e2m1 x e2m1 0.321 -> 0.295 ms,
  // e4m3 x e4m3 0.498 -> 0.489 ms, e4m3 x e2m1 0.449 -> 0.460 ms (slower: by row there). With both
  // layouts conflict-free the mixed pair still runs 2 % faster by row (0.399 against 0.406 ms).
  constexpr bool PK = FA == FB;
  const int base_sa = PK ? L::SA_REGION + (wm * 16 + r16) * 128 : L::SA_REGION + (wm * WM + r16) * SC_CHUNK * 4;
  const int base_sb = PK ? L::SB_REGION + (wn * 16 + r16) * 256 : L::SB_REGION + (wn * WN + r16) * SC_CHUNK * 4;
  const int slot_xa = (r16 >> 1) & 7, slot_xb = (r16 >> 1) & 7, half_xb = (r16 & 1) * 16;
  // v_perm selector: byte q of the low source to byte 0, byte q of the high source to byte 1
  const int sel01 = q | ((4 + q) << 8) | (0x0c << 16) | (0x0c << 24);

  // Copy plan. The per-lane offsets depend only on the lane, the wave and K; the resources
  // describe the unit being copied (rows past it or past N read as zero) and switch from one unit
  // to the next at the first stage whose copies target the next one.
  MxLoadPlan<FA, FB, KS> lp;
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
    lp.srow = (uint32_t)srow;
  }
  auto rsrc_a = [&](const Unit& u, bool live) {
    return make_rsrc((const uint8_t*)p.A + (size_t)u.row0 * rowA, live ? (uint64_t)u.rows * rowA : 0);
  };
  auto rsrc_b = [&](const Unit& u, bool live) {
    return make_rsrc((const uint8_t*)p.B + ((size_t)u.e * N + u.n0) * rowB,
                     live ? (uint64_t)min(BN, N - u.n0) * rowB : 0);
  };
  auto rsrc_scales = [&](const Unit& u, bool live) {
    lp.sa_rsrc = make_rsrc((const uint8_t*)p.a_scales + (size_t)u.row0 * srow, live ? (uint64_t)u.rows * srow : 0);
    lp.sb_rsrc = make_rsrc((const uint8_t*)p.b_scales + ((size_t)u.e * N + u.n0) * srow,
                           live ? (uint64_t)min(BN, N - u.n0) * srow : 0);
  };

  // Scale chunk c of the current unit sits in buffer (cbase + c) & 1.
  int cbase = 0;
  v4f acc[MI][NJ];

  // lane (r16, q) supplies the scale of chunk q: byte q of the row's dword, read as a byte (one LDS
  // read and no shift; measured 3 % faster for e4m3 x e2m1 than a dword read and a shift, both
  // conflict-free)
  // g: 128-K sub-block index of the unit (stage b holds sub-blocks KS b .. KS b + KS - 1)
  auto scale_a = [&](int g, int i) {
    const int so = ((cbase + g / SC_CHUNK) & 1) * SC_BYTES + ((g % SC_CHUNK) ^ slot_xa) * 4;
    return (int)*(const uint8_t*)(smem + base_sa + q + so + i * 16 * SC_CHUNK * 4);
  };
  auto scale_b = [&](int g, int j) {
    const int so = ((cbase + g / SC_CHUNK) & 1) * SC_BYTES + ((g % SC_CHUNK) ^ slot_xb) * 4;
    return (int)*(const uint8_t*)(smem + base_sb + q + so + j * 16 * SC_CHUNK * 4);
  };
  // Packed layout: sub-block g's dwords of the lane's 4 A fragments, or of B fragments 4 h ..
  // 4 h + 3, in one read; pack4 keeps byte q of each (the lane's chunk), fragment f in byte f,
  // which the MFMA then selects.
  auto raw_a = [&](int g) {
    const int so = ((cbase + g / SC_CHUNK) & 1) * SC_BYTES + (((g % SC_CHUNK) ^ slot_xa) * 16);
    return lds_read16(smem + base_sa + so);
  };
  auto raw_b = [&](int g, int h) {
    const int so = ((cbase + g / SC_CHUNK) & 1) * SC_BYTES + (((g % SC_CHUNK) ^ slot_xb) * 32) + (h ? 16 - half_xb : half_xb);
    return lds_read16(smem + base_sb + so);
  };
  auto pack4 = [&](const v4i d) {
    const uint32_t x01 = __builtin_amdgcn_perm((uint32_t)d[1], (uint32_t)d[0], (uint32_t)sel01);
    const uint32_t x23 = __builtin_amdgcn_perm((uint32_t)d[3], (uint32_t)d[2], (uint32_t)sel01);
    return (int)__builtin_amdgcn_perm(x23, x01, 0x05040100u);
  };

  // The stages of unit u into acc. prologue: copy the unit's first stages and scale chunks and
  // wait for them (else the previous unit's last stages copied them). pipe: the last two stages
  // copy the first two of unit nx (zero-byte resources unless nx_live).
  auto run_unit = [&](const Unit& u, const bool prologue, const bool pipe, const Unit& nx, const bool nx_live) {
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (prologue) {
      // copies of the previous unit's last stages may still be in flight into stages reused here
      wait_vmcnt<0>();
      cbase = 0;
      lp.a_rsrc = rsrc_a(u, true);
      lp.b_rsrc = rsrc_b(u, true);
      rsrc_scales(u, true);
      // scale chunks 0 and 1, stage 0 and the B half of stage 1 (its A half goes out in passes 0
      // and 1 of stage 0, as in every stage); stage 0 published
      const LdsBases lb = lds_bases<FA, FB, KS>(smem, wave);
      mx_issue_scales<FA, FB, KS, PK>(lb.ws + L::SA_REGION, lb.ws + L::SB_REGION, lp, 0, wave);
      mx_issue_scales<FA, FB, KS, PK>(lb.ws + L::SA_REGION + SC_BYTES, lb.ws + L::SB_REGION + SC_BYTES, lp, 1, wave);
#pragma unroll
      for (int i = 0; i < L::A_INSTR; i++) mx_copy_a<FA, FB, KS>(lb.wa + L::A_REGION, lp, 0, i);
#pragma unroll
      for (int i = 0; i < L::B_INSTR; i++) mx_copy_b<FA, FB, KS>(lb.wb + L::B_REGION, lp, 0, i);
#pragma unroll
      for (int i = 0; i < L::B_INSTR; i++)
        mx_copy_b<FA, FB, KS>(lb.wb + L::B_REGION + L::B_BYTES, lp, min(1, KB - 1), i);
      wait_vmcnt<0>();
      barrier();
    }

    // A fragments and scales of the stage stay in registers; B fragments and their scales
    // stream through 3-deep queues two fragments ahead
    v8i af[MI], bq[3];
    int sa[MI][KS], sbq[3][KS];     // by row: each fragment's scale in byte 0
    int sa_p[KS], sb_p[KS][2];      // packed: fragment i (A) / j (B) in byte i / j % 4
#pragma unroll
    for (int i = 0; i < MI; i++) {
      af[i] = read_frag<L::RA>(smem + L::A_REGION + i * 16 * L::RA, fa);
      if constexpr (!PK) {
#pragma unroll
        for (int h = 0; h < KS; h++) sa[i][h] = scale_a(h, i);
      }
    }
    bq[0] = read_frag<L::RB>(smem + L::B_REGION, fb);
    bq[1] = read_frag<L::RB>(smem + L::B_REGION + 16 * L::RB, fb);
#pragma unroll
    for (int h = 0; h < KS; h++) {
      if constexpr (PK) {
        sa_p[h] = pack4(raw_a(h));
        sb_p[h][0] = pack4(raw_b(h, 0));
        sb_p[h][1] = pack4(raw_b(h, 1));
      } else {
        sbq[0][h] = scale_b(h, 0);
        sbq[1][h] = scale_b(h, 1);
      }
    }
    // the MFMA of A fragment i, B fragment j, sub-block h with its scales
    auto mma_ij = [&](const v8i& bop, const v8i& aop, const v4f& c, const int i, const int j, const int h) {
      if constexpr (PK) return mma_p<FA, FB>(bop, aop, c, sb_p[h][j / 4], j % 4, sa_p[h], i);
      else return mma<FA, FB>(bop, aop, c, sbq[j % 3][h], sa[i][h]);
    };

    // copies per wave and pass: the A half of a stage over passes 0 and 1, the B half over
    // passes 6 and 7, each after the second or fourth MFMA of the pass
    constexpr int A_PP = L::A_INSTR / 2, B_PP = L::B_INSTR / 2;
    static_assert(A_PP >= 1 && A_PP <= 2 && B_PP >= 1 && B_PP <= 2, "copy schedule");

    // One stage (b) in ring place S = b & 1 (a run-time value: a loop body per place, with the
    // offsets as immediates, needs more registers than the kernel has). Stages of the main loop
    // (TAIL false) copy from the current unit only; the last two (TAIL true) copy the next unit's
    // first stages when piped, else repeat stage KB-1 into a stage that is not read again.
    auto stage = [&](auto tail_tag, const int b) {
      const int S = b & 1;
      constexpr bool TAIL = decltype(tail_tag)::value;
      const int sob = S * L::B_BYTES;                                            // this stage
      const int sna = (S ^ 1) * L::A_BYTES, snb = (S ^ 1) * L::B_BYTES;         // the other one
      const int bn = min(b + 1, KB - 1);
      // copy targets: the A half of stage b+1, the B half of stage b+2
      int kb_a = b + 1, kb_b = min(b + 2, KB - 1);
      const LdsBases lb = lds_bases<FA, FB, KS>(smem, wave);
      if constexpr (TAIL) {
        if (pipe) {
          kb_b = b + 2 - KB;
          if (b == KB - 1) {
            kb_a = 0;
            lp.a_rsrc = rsrc_a(nx, nx_live);
          }
        } else {
          kb_a = bn;
        }
      }
      // passes 0..5: B fragment j against the 4 resident A fragments (with two sub-blocks per
      // stage: sub-block 0 for all four, then sub-block 1, so chained MFMAs are four apart), MFMAs
      // at raised wave priority; B fragment j + 2 is read in two halves (after the first and third
      // MFMA) and its scale after the third. Passes 0 and 1 also copy the A half of stage b+1 into
      // the other stage (freed by the barrier of stage b-1; its B half went out in passes 6 and 7
      // of stage b-1). Each MFMA with what follows it is a scheduling region of its own.
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
          acc[i][j] = mma_ij(sub_op<KS>(bq[j % 3], h), sub_op<KS>(af[i], h), acc[i][j], i, j, h);
          if (h < KS - 1) {
            __builtin_amdgcn_sched_barrier(0);
            continue;
          }
          if (j < 2 && (i & 1) && (i >> 1) < A_PP)
            mx_copy_a<FA, FB, KS>(lb.wa + L::A_REGION + sna, lp, kb_a, j * A_PP + (i >> 1));
          if (j + 2 < NJ && i == 0) lo = lds_read16(smem + L::B_REGION + sob + (j + 2) * 16 * L::RB + fb.off[0]);
          if (j + 2 < NJ && i == 2) {
            if constexpr (L::RB == 128) hi = lds_read16(smem + L::B_REGION + sob + (j + 2) * 16 * L::RB + fb.off[1]);
            if constexpr (!PK) {
#pragma unroll
              for (int h = 0; h < KS; h++) sbn[h] = scale_b(KS * b + h, j + 2);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (j + 2 < NJ) {
          if constexpr (L::RB == 128) bq[(j + 2) % 3] = cat(lo, hi);
          else bq[(j + 2) % 3] = (v8i){lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
          if constexpr (!PK) {
#pragma unroll
            for (int h = 0; h < KS; h++) sbq[(j + 2) % 3][h] = sbn[h];
          }
        }
        // pin the previous pass's MFMAs (complete by now) ahead of this point, so that the
        // compiler does not sink them past the loop's branch
        if (j > 0) {
#pragma unroll
          for (int i = 0; i < MI; i++) asm volatile("" : "+v"(acc[i][j - 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage S fully read (its last read was in pass 5), stage b+1 landed: publish it
      wait_vmcnt<0>();
      wait_lds_reads();
      barrier();
      if constexpr (TAIL) {
        if (pipe && b == KB - 2) lp.b_rsrc = rsrc_b(nx, nx_live);
      }
      // Scale chunks. Chunk c+1 replaces chunk c-1 (read for the last time before the barrier of
      // stage SCS c - 1) while stage SCS c is computed. A unit's first two chunks are loaded before
      // it starts: in its prologue, or piped in the previous unit's stages KB-2 and KB-1 (into the
      // buffers of that unit's chunks n-2 and n-1, n = its chunk count; the last one is read for
      // the last time before the barrier of stage KB-1).
      if constexpr (!TAIL) {
        if (b % SCS == 0 && b > 0 && b / SCS + 1 < nchunks) {
          const int c = b / SCS + 1, cb = ((cbase + c) & 1) * SC_BYTES;
          mx_issue_scales<FA, FB, KS, PK>(lb.ws + L::SA_REGION + cb, lb.ws + L::SB_REGION + cb, lp, c, wave);
        }
      }
      if constexpr (TAIL) {
        if (pipe && b == KB - 2) {
          rsrc_scales(nx, nx_live);
          const int cb = ((cbase + nchunks) & 1) * SC_BYTES;
          mx_issue_scales<FA, FB, KS, PK>(lb.ws + L::SA_REGION + cb, lb.ws + L::SB_REGION + cb, lp, 0, wave);
        }
        if (pipe && b == KB - 1) {
          const int cb = ((cbase + nchunks - 1) & 1) * SC_BYTES;
          mx_issue_scales<FA, FB, KS, PK>(lb.ws + L::SA_REGION + cb, lb.ws + L::SB_REGION + cb, lp, 1, wave);
        }
      }
#pragma unroll
      for (int i = 0; i < MI; i++) asm volatile("" : "+v"(acc[i][NJ - 3]));
      __builtin_amdgcn_sched_barrier(0);
      // packed: the next stage's scale dwords, packed at the end of pass 7 (after this stage's
      // last MFMA that uses the current ones)
      v4i ra_n[KS], rb_n[KS][2];
      if constexpr (PK) {
#pragma unroll
        for (int h = 0; h < KS; h++) {
          ra_n[h] = raw_a(KS * bn + h);
          rb_n[h][0] = raw_b(KS * bn + h, 0);
          rb_n[h][1] = raw_b(KS * bn + h, 1);
        }
      }
      // pass 6 with the first copies of the B half of stage b+2 into stage S
#pragma unroll
      for (int h = 0; h < KS; h++)
#pragma unroll
      for (int i = 0; i < MI; i++) {
        acc[i][NJ - 2] = mma_ij(sub_op<KS>(bq[(NJ - 2) % 3], h), sub_op<KS>(af[i], h), acc[i][NJ - 2], i, NJ - 2, h);
        if ((i & 1) && (i >> 1) < B_PP && h == KS - 1)
          mx_copy_b<FA, FB, KS>(lb.wb + L::B_REGION + sob, lp, kb_b, i >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // pass 7: last B fragment; each A fragment and its scale are refilled from stage b+1
      // right after their MFMA; the rest of the B half of stage b+2; then the first two B
      // fragments of stage b+1 and their scales are read (in the unit's last stage these reads
      // are not used: the next unit reads its first stage afresh)
#pragma unroll
      for (int h = 0; h < KS; h++)
#pragma unroll
      for (int i = 0; i < MI; i++) {
        acc[i][NJ - 1] = mma_ij(sub_op<KS>(bq[(NJ - 1) % 3], h), sub_op<KS>(af[i], h), acc[i][NJ - 1], i, NJ - 1, h);
        if (h < KS - 1) {
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        af[i] = read_frag<L::RA>(smem + L::A_REGION + sna + i * 16 * L::RA, fa);
        if constexpr (!PK) {
#pragma unroll
          for (int h = 0; h < KS; h++) sa[i][h] = scale_a(KS * bn + h, i);
        }
        if ((i & 1) && (i >> 1) < B_PP)
          mx_copy_b<FA, FB, KS>(lb.wb + L::B_REGION + sob, lp, kb_b, B_PP + (i >> 1));
        __builtin_amdgcn_sched_barrier(0);
      }
      bq[0] = read_frag<L::RB>(smem + L::B_REGION + snb, fb);
      bq[1] = read_frag<L::RB>(smem + L::B_REGION + snb + 16 * L::RB, fb);
#pragma unroll
      for (int h = 0; h < KS; h++) {
        if constexpr (PK) {
          sa_p[h] = pack4(ra_n[h]);
          sb_p[h][0] = pack4(rb_n[h][0]);
          sb_p[h][1] = pack4(rb_n[h][1]);
        } else {
          sbq[0][h] = scale_b(KS * bn + h, 0);
          sbq[1][h] = scale_b(KS * bn + h, 1);
        }
      }
#pragma unroll
      for (int i = 0; i < MI; i++) asm volatile("" : "+v"(acc[i][NJ - 2]));
      __builtin_amdgcn_sched_barrier(0);
    };

    int b = 0;
    for (; b + 2 < KB; b++) stage(std::false_type{}, b);
    // the unit's last two stages (or its only one)
    stage(std::true_type{}, b);
    if (b + 1 < KB) stage(std::true_type{}, b + 1);
  };

  // epilogue: lane holds row r16 of each M fragment and, over N fragments 2 jj and 2 jj + 1,
  // columns 32 jj + 8 q .. 32 jj + 8 q + 7 of its 128-column block (see b_col). The stores are
  // not waited for: the next unit's first wait before a barrier covers them.
  auto store_c = [&](const Unit& u) {
#pragma unroll
    for (int i = 0; i < MI; i++) {
      const int mloc = wm * WM + i * 16 + r16;
      if (mloc >= u.rows) continue;
      const size_t crow = (size_t)(u.row0 + mloc) * N;
#pragma unroll
      for (int jj = 0; jj < NJ / 2; jj++) {
        const int col = u.n0 + wn * WN + jj * 32 + q * 8;
        if (col < N) store8<OUT>(C, crow + col, acc[i][2 * jj], acc[i][2 * jj + 1]);
      }
    }
  };

  // The persistent loop: units of items xb, xb + G, ..., one pipeline through all.
  UnitSeq seq;
  seq.L = xb - (int)gridDim.x;
  seq.k = 0;
  Unit cu, nx = {0, 0, 0, 0};
  bool have = next_unit(p, tm, n_blocks, items, seq, cu);
  bool have_next = have && next_unit(p, tm, n_blocks, items, seq, nx);
  for (bool first = true; have; first = false) {
    if (!first && !piped) barrier();   // every wave is past its last LDS read of the previous unit
    run_unit(cu, first || !piped, piped, nx, have_next && piped);
    store_c(cu);
    if (!have_next) break;
    cbase = (cbase + nchunks) & 1;
    cu = nx;
    have_next = next_unit(p, tm, n_blocks, items, seq, nx);
  }
}

template <int FA, int FB, int KS = 1>
hipError_t launch_fmt(const GemmArgs& a, int out, hipStream_t stream, dim3 grid, int n_blocks) {
  dim3 block(NTHREADS);
  const int32_t* eids = a.expert_ids;
  const int32_t* toffs = a.tile_offsets;
  void* c = a.C;
  switch (out) {
    case kOutF32: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutF32, KS>), grid, block, 0, stream, a, n_blocks, eids, toffs, c); break;
    case kOutBF16: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutBF16, KS>), grid, block, 0, stream, a, n_blocks, eids, toffs, c); break;
    case kOutF16: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutF16, KS>), grid, block, 0, stream, a, n_blocks, eids, toffs, c); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx(const GemmArgs& a0, int fmt_a, int fmt_b, int out, hipStream_t stream) {
  const int n_blocks = (a0.N + BN - 1) / BN;
  const long long blocks = (long long)((a0.num_tiles + 1) / 2) * n_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0LL) return hipErrorInvalidValue;
  // persistent grid: one workgroup per compute unit (the LDS ring allows one), fewer when there
  // are fewer items; a multiple of 8 for the XCD-aware order. Work order in groups of 8
  // super-tiles, or 1 when there are at most 8 column blocks (groups of 4, as the blockwise
  // kernel uses, measured 1 % slower for e4m3 x e4m3 and the same for e2m1 x e2m1).
  const dim3 grid(grid_for(blocks < a0.num_cus ? blocks : a0.num_cus));
  GemmArgs a = a0;
  a.group_m = n_blocks <= 8 ? 1 : 8;
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
