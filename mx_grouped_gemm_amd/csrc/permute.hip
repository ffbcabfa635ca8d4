// Activation quantisation and token permutation into the grouped GEMM's A operand (gfx950).
//
// The grouped GEMM of the Modular MAX page "promote_accumulators" (section Args) reads A with
// its rows grouped by expert and one fp32 scale per row per 128 K-elements. These kernels build
// that input from token activations and top-k picks:
//   route_counts  picks per expert (a histogram of the top-k ids)
//   permute_rank  row of every pick: expert e's picks fill rows expert_offsets[e].. in token
//                 order; the rest of each group (its padding) is zeroed with scale 1
//   quantize      per token row and 128-block: s = amax / 448, q = rne_e4m3(clamp(x / s)),
//                 both divisions in fp32; the row goes to each of its top_k destinations
// All three are HBM- or latency-bound; none needs the matrix units.
#include "common.h"
#include "launch.h"

namespace bsg {
namespace {

constexpr int kHistThreads = 1024;
constexpr int kHistPerBlock = 8192;      // picks per histogram workgroup

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Workgroup histogram in LDS over kHistPerBlock picks, then one global add per expert.
__global__ __launch_bounds__(kHistThreads) void route_counts_kernel(const int32_t* __restrict__ ids,
                                                                    int n, int E, int32_t* counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += kHistThreads) hist[e] = 0;
  __syncthreads();
  const long long base = (long long)blockIdx.x * kHistPerBlock;
  for (int k = threadIdx.x; k < kHistPerBlock; k += kHistThreads) {
    const long long i = base + k;
    if (i < n) {
      const int e = ids[i];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kHistThreads)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

constexpr int kRankThreads = 1024, kRankWaves = kRankThreads / kWave;
constexpr int kRankPer = 16;             // consecutive picks per thread and chunk (four 16-byte loads)
constexpr int kRankChunk = kRankThreads * kRankPer;

// Exclusive prefix over the wave of small per-lane counts (0 .. 31) from five ballots.
__device__ __forceinline__ int wave_prefix5(int c, int lane) {
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int pre = 0;
#pragma unroll
  for (int bit = 0; bit < 5; bit++)
    pre += __popcll(__ballot((c >> bit) & 1) & below) << bit;
  return pre;
}

// The thread's kRankPer picks of the chunk starting at c0 (-1 past the end).
__device__ __forceinline__ void load_picks(const int32_t* __restrict__ ids, long long n, long long i0,
                                           int (&id)[kRankPer]) {
  if (i0 + kRankPer <= n && ((uintptr_t)ids & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kRankPer / 4; q++) {
      const v4i v = *(const v4i*)(ids + i0 + 4 * q);
      id[4 * q] = v[0]; id[4 * q + 1] = v[1]; id[4 * q + 2] = v[2]; id[4 * q + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRankPer; k++) id[k] = i0 + k < n ? ids[i0 + k] : -1;
  }
}

// Workgroups P e .. P e + P - 1: rows of expert e's picks, in pick order (token-major), and its
// padding rows. All P scan the picks alike (the count of e's picks fixes where its padding
// starts); the first writes the picks' rows and each zeroes every P-th padding row, so that the
// padding of one expert (up to 127 rows of K codes) is not written by one compute unit alone
// (with P = 1 that took 11 of 38 us on the 32-expert activations). Each chunk's picks are loaded
// one chunk ahead, so a chunk costs its ballots and one barrier.
__global__ __launch_bounds__(kRankThreads) void permute_rank_kernel(
    const int32_t* __restrict__ ids, int n, int E, int P, const int32_t* __restrict__ expert_offsets,
    int M, int K, int32_t* __restrict__ dest, uint8_t* __restrict__ qa, float* __restrict__ a_scales) {
  __shared__ int wave_tot[2][kRankWaves];
  const int e = blockIdx.x / P, part = blockIdx.x % P, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long off = expert_offsets[e];
  int running = 0;
  int nxt[kRankPer];
  load_picks(ids, n, (long long)tid * kRankPer, nxt);
  for (long long c0 = 0, it = 0; c0 < n; c0 += kRankChunk, it++) {
    const long long i0 = c0 + (long long)tid * kRankPer;
    int id[kRankPer];
#pragma unroll
    for (int k = 0; k < kRankPer; k++) id[k] = nxt[k];
    if (c0 + kRankChunk < n) load_picks(ids, n, i0 + kRankChunk, nxt);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kRankPer; k++) {
      cnt += id[k] == e;
      // picks whose id is outside the experts are marked by workgroup 0
      if (e == 0 && part == 0 && i0 + k < n && (id[k] < 0 || id[k] >= E)) dest[i0 + k] = -1;
    }
    const int pre = wave_prefix5(cnt, lane);
    int* tot = wave_tot[it & 1];
    if (lane == 63) tot[wave] = pre + cnt;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; w++) {
      const int t = tot[w];
      before += w < wave ? t : 0;
      total += t;
    }
    // the thread's matches in pick order, one store per match: the loop runs as many times as
    // the most matches of a lane in the wave, not once per pick
    if (part == 0) {
      uint32_t mask = 0;
#pragma unroll
      for (int k = 0; k < kRankPer; k++) mask |= (uint32_t)(id[k] == e) << k;
      int r = running + before + pre;
      while (mask) {
        const int k = __builtin_ctz(mask);
        mask &= mask - 1;
        const long long row = off + r;
        dest[i0 + k] = row >= 0 && row < M ? (int32_t)row : -1;
        r++;
      }
    }
    running += total;
  }
  // padding rows of the group: zero codes, scale 1
  // (offsets are clamped into [0, M]: rows outside qa are never written)
  const long long lo = max(0LL, min(off + running, (long long)M));
  const long long hi = min((long long)expert_offsets[e + 1], (long long)M);
  const int KB = K / 128, per_row = K / 16;
  for (long long rr = lo + part; rr < hi; rr += P) {
    for (int k = tid; k < per_row; k += kRankThreads) *(v4i*)(qa + rr * K + 16 * k) = (v4i){0, 0, 0, 0};
    for (int k = tid; k < KB; k += kRankThreads) a_scales[rr * KB + k] = 1.0f;
  }
}

// Round-to-nearest-even of a finite fp32 value with |y| <= 448 onto e4m3fn (OFP8 layout).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y), sign = (u >> 31) << 7, a = u & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {                          // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    uint32_t e = (a >> 23) - 127 + 7, keep = (a >> 20) & 7;
    const uint32_t rem = a & 0xfffffu, half = 0x80000u;
    keep += (rem > half) || (rem == half && (keep & 1));
    if (keep == 8) { keep = 0; e++; }
    code = (e << 3) | keep;
  }
  return code | sign;
}

template <typename T> __device__ __forceinline__ void load16(const T* p, float (&v)[16]);
template <> __device__ __forceinline__ void load16<float>(const float* p, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const float4 a = *(const float4*)(p + 4 * q);
    v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
  }
}
template <> __device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const v4i a = *(const v4i*)(p + 8 * q);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[8 * q + 2 * k] = __uint_as_float((uint32_t)a[k] << 16);
      v[8 * q + 2 * k + 1] = __uint_as_float((uint32_t)a[k] & 0xffff0000u);
    }
  }
}

constexpr int kQuantWaves = 4;

template <typename T>
__device__ __forceinline__ void load_chunk(const T* __restrict__ row, int K, int k0, float (&v)[16]) {
  if (k0 < K) load16<T>(row + k0, v);
  else {
#pragma unroll
    for (int k = 0; k < 16; k++) v[k] = 0.f;
  }
}

// One wave per token: 1024 elements per step, 8 lanes (16 elements each) per 128-block; each
// destination row gets one 16-byte store per lane. The next step's elements are loaded before
// this step's stores go out. The codes are stored non-temporal (streamed past the caches:
// 1 GB of grouped rows written once); measured on the 32-expert activations (16384 tokens x 8
// picks, K 7168), one call 0.330 -> 0.267 ms. Non-temporal loads of the activations and
// non-temporal scale stores made the call slower (0.317 ms) and are not used.
template <typename T>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_kernel(
    const T* __restrict__ x, int tokens, int top_k, int K, const int32_t* __restrict__ dest,
    uint8_t* __restrict__ qa, float* __restrict__ a_scales) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const int KB = K / 128;
  const T* row = x + (long long)t * K;
  int rows[8];
  for (int j0 = 0; j0 < top_k; j0 += 8) {
    const int nj = min(8, top_k - j0);
#pragma unroll
    for (int j = 0; j < 8; j++) rows[j] = j < nj ? dest[(long long)t * top_k + j0 + j] : -1;
    float vn[16];
    load_chunk<T>(row, K, 16 * lane, vn);
    for (int c = 0; c < K; c += 1024) {
      const int k0 = c + 16 * lane;
      const bool live = k0 < K;                  // K is a multiple of 128: whole blocks drop out
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; k++) v[k] = vn[k];
      if (c + 1024 < K) load_chunk<T>(row, K, k0 + 1024, vn);
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 16; k++) amax = fmaxf(amax, fabsf(v[k]));
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 8));
      const float s = amax > 0.f ? amax / 448.0f : 1.0f;
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 16; k++) {
        const float y = fminf(fmaxf(v[k] / s, -448.0f), 448.0f);
        w[k / 4] |= e4m3_rne(y) << (8 * (k % 4));
      }
      if (live) {
        const v4i packed = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const int r = rows[j];
          if (r < 0) continue;
          __builtin_nontemporal_store(packed, (v4i*)(qa + (long long)r * K + k0));
          if ((lane & 7) == 0) a_scales[(long long)r * KB + k0 / 128] = s;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_route_counts(const int32_t* ids, int n, int E, int32_t* counts, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, counts, E);
  if (n > 0) {
    const int blocks = (int)(((long long)n + kHistPerBlock - 1) / kHistPerBlock);
    hipLaunchKernelGGL(route_counts_kernel, dim3(blocks), dim3(kHistThreads), E * sizeof(int), stream, ids,
                       n, E, counts);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_permute(const void* x, int x_f32, const int32_t* ids, int tokens, int top_k,
                                   int K, int E, const int32_t* expert_offsets, int M, int32_t* dest,
                                   uint8_t* qa, float* a_scales, hipStream_t stream) {
  const int n = tokens * top_k;
  // workgroups per expert: enough to spread the padding over about 256 workgroups
  const int P = E >= 256 ? 1 : 256 / E;
  hipLaunchKernelGGL(permute_rank_kernel, dim3(E * P), dim3(kRankThreads), 0, stream, ids, n, E, P,
                     expert_offsets, M, K, dest, qa, a_scales);
  if (tokens > 0) {
    const dim3 grid((tokens + kQuantWaves - 1) / kQuantWaves), block(kQuantWaves * kWave);
    if (x_f32)
      hipLaunchKernelGGL(quantize_kernel<float>, grid, block, 0, stream, (const float*)x, tokens, top_k, K,
                         dest, qa, a_scales);
    else
      hipLaunchKernelGGL(quantize_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t*)x, tokens,
                         top_k, K, dest, qa, a_scales);
  }
  return hipGetLastError();
}

}  // namespace bsg
