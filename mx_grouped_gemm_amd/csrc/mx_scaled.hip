// MX block-scaled GEMM for gfx950 (MI355X): e4m3 / e2m1 elements, one e8m0 scale per 32
// K-elements per row of A and per row of B (the MX variant of the Triton Gluon page
// "Overlapping Accumulator Block-Scaled Matrix Multiplication": scales applied inside the
// matrix instruction, as its async_mma_scaled_impl does with tcgen05_mma_scaled; reference
// result A_ref @ B_ref^T of its make_problem).
//
// CDNA4 mapping: v_mfma_scale_f32_32x32x64_f8f6f4 takes per-lane e8m0 scales for the
// 32-element K chunk each lane supplies, so no software promotion is needed and the fp32
// accumulator chains through the instruction. Same block structure as the blockwise kernel:
// 8 waves, 128 x 256 tile, 2 x 2 fragments of 32 x 32 per wave, 3-stage LDS ring filled by
// direct global->LDS loads; per stage each row's four scale bytes (128 K) are one dword
// staged next to the tiles. Supports the tile map (grouped) and one dense group.
#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int NWAVES = 8, NTHREADS = NWAVES * kWave;
constexpr int STAGES = 3;

// element format codes of the f8f6f4 instruction: 0 = e4m3, 4 = e2m1
template <int F> struct Elem;
template <> struct Elem<1> { static constexpr int kRowBytes = 128; static constexpr int kCode = 0; };
template <> struct Elem<2> { static constexpr int kRowBytes = 64; static constexpr int kCode = 4; };

template <int FA, int FB>
struct Layout {
  static constexpr int RA = Elem<FA>::kRowBytes, RB = Elem<FB>::kRowBytes;
  static constexpr int A_BYTES = BM * RA;
  static constexpr int B_BYTES = BN * RB;
  static constexpr int AS_OFF = A_BYTES + B_BYTES;              // dword of 4 scales per A row
  static constexpr int BS_OFF = AS_OFF + BM * 4;                // dword per B row
  static constexpr int STAGE_BYTES = BS_OFF + BN * 4;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // 1 KiB instructions per wave per stage: A rows, B rows; plus one A-scale and one B-scale load
  static constexpr int A_INSTR = A_BYTES / 1024 / NWAVES;
  static constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;
  static constexpr int LOADS = A_INSTR + B_INSTR + 2;
  static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small for the load split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int ROWB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (ROWB == 128) return swz8(r); else return swz4(r);
}

// Fragment operand for one 64-wide K half (K chunks 2kh and 2kh+1 of 32 elements each).
// The scale supplied by lane l covers row l % 32, chunk l / 32 of the half. For e2m1 the lane
// holds that whole chunk (16 bytes). For e4m3 the instruction takes bytes 0..15 of every lane
// from the first chunk and bytes 16..31 from the second, lane halves kq = 0 / 1 splitting each
// chunk: so lane kq reads K [16 kq, 16 kq + 16) of both chunks.
template <int ROWB>
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int kh, int kq) {
  if constexpr (ROWB == 128) {
    const int c0 = kh * 4 + kq, c1 = kh * 4 + 2 + kq;
    return cat(lds_read16(tile + r * ROWB + ((c0 ^ swz8(r)) * 16)),
               lds_read16(tile + r * ROWB + ((c1 ^ swz8(r)) * 16)));
  } else {
    const int c = kh * 2 + kq;
    const v4i v = lds_read16(tile + r * ROWB + ((c ^ swz4(r)) * 16));
    return (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
  }
}

template <int FA, int FB>
struct MxLoadPlan {
  const uint8_t* a_src[Layout<FA, FB>::A_INSTR];
  const uint8_t* b_src[Layout<FA, FB>::B_INSTR];
  const uint8_t* sa_src;
  const uint8_t* sb_src;
  int a_dst[Layout<FA, FB>::A_INSTR], b_dst[Layout<FA, FB>::B_INSTR], sa_dst, sb_dst;
};

template <int FA, int FB>
__device__ __forceinline__ void mx_issue(uint8_t* dst, const MxLoadPlan<FA, FB>& lp, int kb, int lane) {
  using L = Layout<FA, FB>;
#pragma unroll
  for (int i = 0; i < L::A_INSTR; i++) g2lds16(lp.a_src[i] + (size_t)kb * L::RA, as_lds(dst + lp.a_dst[i]));
#pragma unroll
  for (int i = 0; i < L::B_INSTR; i++) g2lds16(lp.b_src[i] + (size_t)kb * L::RB, as_lds(dst + lp.b_dst[i]));
  if (lane < 16) g2lds4(lp.sa_src + (size_t)kb * 4, as_lds(dst + lp.sa_dst));
  if (lane < 32) g2lds4(lp.sb_src + (size_t)kb * 4, as_lds(dst + lp.sb_dst));
}

// One K block of 128: copies of K block kb_next into `nxt` (if requested), then four pairs of
// scaled MFMAs on the operands in `cur`. The two stages are distinct (see the blockwise kernel).
template <int FA, int FB>
__device__ __forceinline__ void mx_step(const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt,
                                        const MxLoadPlan<FA, FB>& lp, bool issue, int kb_next,
                                        int lane, int wm, int wn, v16f (&acc)[2][2]) {
  using L = Layout<FA, FB>;
  if (issue) mx_issue<FA, FB>(nxt, lp, kb_next, lane);
  const int fr = lane & 31, kq = lane >> 5;
  v8i af[2][2], bf[2][2];
  int sa[2], sb[2];
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int ra = wm * 64 + f * 32 + fr, rb = wn * 64 + f * 32 + fr;
#pragma unroll
    for (int kh = 0; kh < 2; kh++) {
      af[f][kh] = read_frag<L::RA>(cur, ra, kh, kq);
      bf[f][kh] = read_frag<L::RB>(cur + L::A_BYTES, rb, kh, kq);
    }
    // byte j of the row's dword is the scale of K chunk j (32 elements); lanes of the upper
    // half supply chunks 1 and 3, so their dword is shifted by one byte and bytes 0 / 2 are
    // selected for the two K halves.
    sa[f] = (int)(*(const uint32_t*)(cur + L::AS_OFF + ra * 4) >> (8 * kq));
    sb[f] = (int)(*(const uint32_t*)(cur + L::BS_OFF + rb * 4) >> (8 * kq));
  }
#pragma unroll
  for (int mi = 0; mi < 2; mi++)
#pragma unroll
    for (int ni = 0; ni < 2; ni++) {
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          bf[ni][0], af[mi][0], acc[mi][ni], Elem<FB>::kCode, Elem<FA>::kCode, 0, sb[ni], 0, sa[mi]);
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          bf[ni][1], af[mi][1], acc[mi][ni], Elem<FB>::kCode, Elem<FA>::kCode, 2, sb[ni], 2, sa[mi]);
    }
}

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(NTHREADS, 1) void mx_kernel(GemmArgs p, int n_blocks) {
  using L = Layout<FA, FB>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int t, nb;
  if (!work_item(p.num_tiles, n_blocks, 8, t, nb)) return;
  const int n0 = nb * BN;
  const TileRows tr = tile_rows(p.expert_ids, p.tile_offsets, t, p.M, BM, p.num_experts);
  if (tr.rows <= 0) return;
  const int e = tr.expert, row0 = tr.row0, rows = tr.rows;
  const int N = p.N, KB = p.K / BK;
  const size_t K = (size_t)p.K;
  const size_t rowA = K * L::RA / BK, rowB = K * L::RB / BK;   // bytes per full row
  const size_t srow = K / 32;                                   // scale bytes per row
  const uint8_t* A = (const uint8_t*)p.A;
  const uint8_t* Be = (const uint8_t*)p.B + (size_t)e * N * rowB;
  const uint8_t* SA = (const uint8_t*)p.a_scales;
  const uint8_t* SBe = (const uint8_t*)p.b_scales + (size_t)e * N * srow;

  // ---- load plan: a 1 KiB instruction covers 1024 / rowbytes rows ----
  constexpr int CA = L::RA / 16, CB = L::RB / 16;              // chunks per LDS row
  MxLoadPlan<FA, FB> lp;
#pragma unroll
  for (int i = 0; i < L::A_INSTR; i++) {
    const int first = (wave * L::A_INSTR + i) * (1024 / L::RA);
    const int r = first + lane / CA, slot = lane % CA;
    const int gr = row0 + min(r, rows - 1);
    lp.a_src[i] = A + (size_t)gr * rowA + (size_t)((slot ^ swz<L::RA>(r)) * 16);
    lp.a_dst[i] = first * L::RA;
  }
#pragma unroll
  for (int i = 0; i < L::B_INSTR; i++) {
    const int first = (wave * L::B_INSTR + i) * (1024 / L::RB);
    const int r = first + lane / CB, slot = lane % CB;
    const int gn = min(n0 + r, N - 1);
    lp.b_src[i] = Be + (size_t)gn * rowB + (size_t)((slot ^ swz<L::RB>(r)) * 16);
    lp.b_dst[i] = L::A_BYTES + first * L::RB;
  }
  // scales: wave w stages A rows 16w + (lane & 15) and B rows 32w + (lane & 31)
  lp.sa_src = SA + (size_t)(row0 + min(wave * 16 + (lane & 15), rows - 1)) * srow;
  lp.sb_src = SBe + (size_t)min(n0 + wave * 32 + (lane & 31), N - 1) * srow;
  lp.sa_dst = L::AS_OFF + wave * 16 * 4;
  lp.sb_dst = L::BS_OFF + wave * 32 * 4;

  const int wm = wave & 1, wn = wave >> 1;
  const int fr = lane & 31, kq = lane >> 5;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = (v16f){};

  mx_issue<FA, FB>(smem, lp, 0, lane);
  if (KB > 1) mx_issue<FA, FB>(smem + L::STAGE_BYTES, lp, 1, lane);

  for (int kb = 0; kb < KB; kb++) {
    const int s = kb % STAGES, s2 = (kb + 2) % STAGES;
    if (kb + 1 < KB) wait_vmcnt<L::LOADS>(); else wait_vmcnt<0>();
    barrier();                                                 // stage s landed; stage s2 free
    mx_step<FA, FB>(smem + s * L::STAGE_BYTES, smem + s2 * L::STAGE_BYTES, lp, kb + 2 < KB, kb + 2,
                    lane, wm, wn, acc);
  }

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

template <int FA, int FB>
hipError_t launch_fmt(const GemmArgs& a, int out, hipStream_t stream, dim3 grid, int n_blocks) {
  dim3 block(NTHREADS);
  switch (out) {
    case kOutF32: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutF32>), grid, block, 0, stream, a, n_blocks); break;
    case kOutBF16: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutBF16>), grid, block, 0, stream, a, n_blocks); break;
    case kOutF16: hipLaunchKernelGGL((mx_kernel<FA, FB, kOutF16>), grid, block, 0, stream, a, n_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx(const GemmArgs& a, int fmt_a, int fmt_b, int out, hipStream_t stream) {
  const int n_blocks = (a.N + BN - 1) / BN;
  const long long blocks = (long long)a.num_tiles * n_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0LL) return hipErrorInvalidValue;
  const dim3 grid(grid_for(blocks));
  if (fmt_a == 1 && fmt_b == 1) return launch_fmt<1, 1>(a, out, stream, grid, n_blocks);
  if (fmt_a == 1 && fmt_b == 2) return launch_fmt<1, 2>(a, out, stream, grid, n_blocks);
  if (fmt_a == 2 && fmt_b == 1) return launch_fmt<2, 1>(a, out, stream, grid, n_blocks);
  if (fmt_a == 2 && fmt_b == 2) return launch_fmt<2, 2>(a, out, stream, grid, n_blocks);
  return hipErrorInvalidValue;
}

}  // namespace bsg
