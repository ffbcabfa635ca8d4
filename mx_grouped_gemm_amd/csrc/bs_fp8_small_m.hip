// Grouped blockwise-FP8 GEMM for M-tiles of few rows (decode-sized expert groups), gfx950.
//
// Same operation as bs_fp8_grouped.hip (per 128-K block a fresh fp32 partial, promoted with
// a_scales[row, kb] * b_scales[e, col / 128, kb]; the "promote_accumulators" page of Modular
// MAX, description paragraph and section Args), scheduled for M-tiles that hold few rows: when
// each expert receives a handful of tokens, a 256-row block tile is mostly padding. Here a work
// item is one 128-row M-tile x 256 columns, B is streamed once per item, and the matrix work
// stops at the tile's last real 16-row fragment.
//
//  * 8 waves, each owning 32 columns x the tile's rows as 8 x 2 fragments of 16 x 16; fragments
//    past the last row are skipped (a wave-uniform test). The MFMA is the large-tile kernel's
//    (v_mfma_f32_16x16x128_f8f6f4, B rows as the first operand) with the same promotion
//    order, so results are bitwise identical to it.
//  * a 3-stage LDS ring (50 KiB per stage: 256 B rows and 128 A rows of 128 bytes, XOR-swizzled,
//    plus scales) filled by buffer -> LDS copies two blocks ahead; every wave issues the same 7
//    copies per block (4 of B, 2 of A, 1 of scales), so one vmcnt count waits for a block. A rows
//    past the tile read as zero without touching memory.
//  * scales ride in the stage: the B scales of the two 128-column blocks (waves 0, 1) and the
//    A scales of rows 0-63 and 64-127 (waves 2, 3); waves 4-7 repeat those into spare slots.
#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = 256, BK = 128, BM = 128;
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int WN = BN / NWAVES;                   // 32 columns per wave
constexpr int MI = BM / 16, NJ = WN / 16;         // 8 x 2 fragments
constexpr int STAGES = 3;
constexpr int B_BYTES = BN * BK, A_BYTES = BM * BK;   // 32 KiB, 16 KiB
constexpr int S_BYTES = NWAVES * 256;                 // one 256-byte scale copy per wave
constexpr int STAGE = B_BYTES + A_BYTES + S_BYTES;
constexpr int LDS_BYTES = STAGES * STAGE;             // 153600 of 160 KiB
constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;      // 4
constexpr int A_INSTR = A_BYTES / 1024 / NWAVES;      // 2
constexpr int COPIES_PER_BLOCK = B_INSTR + A_INSTR + 1;

__device__ __forceinline__ v4f mma(const v8i& b, const v8i& a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                          0, 0, 0);
}

struct Plan {
  __amdgpu_buffer_rsrc_t a, b, s;     // s: this wave's scale source (B or A scales)
  uint32_t b_voff[B_INSTR], a_voff[A_INSTR], s_voff;
};

constexpr int kCachePolicyNT = 2;   // cache-policy operand of the buffer load: the nt bit

// Copies of K block kb into stage `st`: B rows 32 w + 8 i + lane / 8, A rows 16 w + 8 i + lane / 8,
// and this wave's scale copy into slot w of the stage's scale area. The B copies carry the
// non-temporal cache policy (the `nt` bit): with one tile per expert each B byte is read once,
// and streaming it took the 128-token decode launch (compact layout) from 167.7 to 162.4 us.
__device__ __forceinline__ void issue_block(uint8_t* smem, const Plan& pl, int kb, int st, int wave) {
  kb = __builtin_amdgcn_readfirstlane(kb);
  uint8_t* base = smem + st * STAGE;
  const uint32_t koff = (uint32_t)kb * BK;
#pragma unroll
  for (int i = 0; i < B_INSTR; i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pl.b, as_lds(base + (wave * B_INSTR + i) * 1024), 16, pl.b_voff[i],
                                             koff, 0, kCachePolicyNT);
#pragma unroll
  for (int i = 0; i < A_INSTR; i++)
    buf2lds16(pl.a, pl.a_voff[i], koff, as_lds(base + B_BYTES + (wave * A_INSTR + i) * 1024));
  // a B scale is one float for every lane (offset from kb alone); an A scale is one per lane (row)
  buf2lds4(pl.s, pl.s_voff, (uint32_t)kb * 4, as_lds(base + B_BYTES + A_BYTES + wave * 256));
}

template <int OUT>
__global__ __launch_bounds__(NTHREADS, 1) void bw_fp8_small_m_kernel(GemmArgs p, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x / n_blocks, nb = blockIdx.x % n_blocks;
  const TileRows tr = tile_rows(p.expert_ids, p.tile_offsets, t, p.M, BM, p.num_experts);
  if (tr.rows <= 0) return;
  const int e = __builtin_amdgcn_readfirstlane(tr.expert);
  const int row0 = __builtin_amdgcn_readfirstlane(tr.row0), rows = __builtin_amdgcn_readfirstlane(tr.rows);
  const int nfrag = (rows + 15) / 16;               // live row fragments
  const int N = p.N, KB = p.K / BK, n0 = nb * BN;
  const size_t K = (size_t)p.K;
  const int r16 = lane & 15, q = lane >> 4, lrow = lane >> 3, slot = lane & 7;

  Plan pl;
  pl.b = make_rsrc((const uint8_t*)p.B + ((size_t)e * N + n0) * K, (uint64_t)min(BN, N - n0) * K);
  pl.a = make_rsrc((const uint8_t*)p.A + (size_t)row0 * K, (uint64_t)rows * K);
#pragma unroll
  for (int i = 0; i < B_INSTR; i++) {
    const int r = wave * 32 + i * 8 + lrow;         // swz8(r) = lrow ^ (i & 1)
    pl.b_voff[i] = (uint32_t)(r * K + ((slot ^ lrow ^ (i & 1)) * 16));
  }
#pragma unroll
  for (int i = 0; i < A_INSTR; i++) {
    const int r = wave * 16 + i * 8 + lrow;         // swz8(r) = lrow ^ (i & 1)
    pl.a_voff[i] = (uint32_t)(r * K + ((slot ^ lrow ^ (i & 1)) * 16));
  }
  // scale copies: wave w & 3 = 0 / 1: B scale of column block 0 / 1 (all lanes one float);
  // 2 / 3: A scales of rows 0-63 / 64-127 (lane = row; rows past the tile read zero)
  if ((wave & 3) < 2) {
    const int cb = min(n0 / 128 + (wave & 1), N / 128 - 1);
    pl.s = make_rsrc((const float*)p.b_scales + ((size_t)e * (N / 128) + cb) * KB, (uint64_t)KB * 4);
    pl.s_voff = 0;
  } else {
    pl.s = make_rsrc((const float*)p.a_scales + (size_t)row0 * KB, (uint64_t)rows * KB * 4);
    pl.s_voff = (uint32_t)(((wave & 1) * 64 + lane) * KB * 4);
  }

  // per-lane LDS read bases (row r16 of fragment 0; chunks 2q and 2q+1 of the 128-byte row)
  const int sw = (r16 & 7) ^ ((r16 >> 3) & 1);
  int base_a[2], base_b[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int chunk = ((2 * q + h) ^ sw) * 16;
    base_a[h] = B_BYTES + r16 * BK + chunk;
    base_b[h] = (wave * WN + r16) * BK + chunk;
  }
  const int s_bs = B_BYTES + A_BYTES + (wave >> 2) * 256;   // B scale of this wave's columns
  const int s_as = B_BYTES + A_BYTES + 2 * 256;              // A scales: rows 0-63, then 64-127

  v4f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; i++)
#pragma unroll
    for (int j = 0; j < NJ; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // prologue: blocks 0 and 1 in flight (past the end they repeat block KB-1 into stages that
  // are not read before they are refilled)
#pragma unroll
  for (int s = 0; s < STAGES - 1; s++) issue_block(smem, pl, min(s, KB - 1), s, wave);

  for (int b = 0; b < KB; b++) {
    const int st = b % STAGES;
    // block b has landed once at most the copies of block b+1 are outstanding
    wait_vmcnt<COPIES_PER_BLOCK>();
    barrier();                                   // ... for every wave; stage (b+2) % 3 is free
    issue_block(smem, pl, min(b + STAGES - 1, KB - 1), (b + STAGES - 1) % STAGES, wave);
    const uint8_t* sp = smem + st * STAGE;
    v8i bf[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++)
      bf[j] = cat(lds_read16(sp + base_b[0] + j * 16 * BK), lds_read16(sp + base_b[1] + j * 16 * BK));
    const float bs = *(const float*)(sp + s_bs);
#pragma unroll
    for (int i = 0; i < MI; i++) {
      if (i < nfrag) {
        const v8i af = cat(lds_read16(sp + base_a[0] + i * 16 * BK), lds_read16(sp + base_a[1] + i * 16 * BK));
        const float sc = *(const float*)(sp + s_as + (16 * i + r16) * 4) * bs;
#pragma unroll
        for (int j = 0; j < NJ; j++) acc[i][j] += mma(bf[j], af) * sc;
      }
    }
  }
  wait_vmcnt<0>();

  // epilogue: lane holds row r16 of each fragment and columns 4 q .. 4 q + 3
#pragma unroll
  for (int i = 0; i < MI; i++) {
    const int mloc = i * 16 + r16;
    if (mloc >= rows) continue;
    const size_t crow = (size_t)(row0 + mloc) * N;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int col = n0 + wave * WN + j * 16 + q * 4;
      if (col < N) store4<OUT>(p.C, crow + col, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
}

}  // namespace

hipError_t launch_blockwise_fp8_small_m(const GemmArgs& a, int out, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long blocks = (long long)a.num_tiles * n_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(NTHREADS);
  switch (out) {
    case kOutF32: hipLaunchKernelGGL(bw_fp8_small_m_kernel<kOutF32>, grid, block, 0, stream, a, n_blocks); break;
    case kOutBF16: hipLaunchKernelGGL(bw_fp8_small_m_kernel<kOutBF16>, grid, block, 0, stream, a, n_blocks); break;
    case kOutF16: hipLaunchKernelGGL(bw_fp8_small_m_kernel<kOutF16>, grid, block, 0, stream, a, n_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsg
