// C ABI of the grouped block-scaled GEMM library: argument validation, device check and
// dispatch to the gfx950 kernels. Declarations and contracts: include/bsgemm.h.
#include "../../include/bsgemm.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
// per-device cache: 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_num_cus[kMaxDevices];

// Checks that the current device is a gfx950; on success stores its compute-unit count in
// *num_cus (if given).
int check_device(int* num_cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return BSG_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) return BSG_ERR_DEVICE;
  int known = g_arch_ok[dev].load(std::memory_order_acquire);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return BSG_ERR_DEVICE;
    }
    known = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_num_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                         std::memory_order_relaxed);
    g_arch_ok[dev].store(known, std::memory_order_release);
  }
  if (num_cus) *num_cus = g_num_cus[dev].load(std::memory_order_relaxed);
  return known == 1 ? BSG_OK : BSG_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Scratch of bsgemm_grouped_noalloc: the workspace of the split-K schedule (4 KiB of flags, then
// 64 fp32 partial tiles of 256 x 256) as a device array the library holds for the process's
// lifetime on every device it runs on. Host code uses its device address per device, never the
// array's host-side name.
constexpr size_t kScratchBytes = 4096 + 64 * (size_t)256 * 256 * 4;   // 16 MiB + 4 KiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of scratch on device dev (the current device), looked up once per device.
void* scratch_ptr(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" const char* bsgemm_status_string(int status) {
  switch (status) {
    case BSG_OK: return "ok";
    case BSG_ERR_NULL: return "a required pointer is NULL";
    case BSG_ERR_SHAPE: return "invalid size (negative, too large, or not a required multiple)";
    case BSG_ERR_ALIGN: return "pointer not aligned as required";
    case BSG_ERR_FMT: return "unsupported fmt combination";
    case BSG_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case BSG_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int bsgemm_build_tiles(const int32_t* counts, int32_t num_experts, int32_t num_tiles,
                                  int32_t padded, int32_t* expert_offsets, int32_t* tile_offsets,
                                  int32_t* expert_ids, void* stream) {
  if (num_experts < 1 || num_experts > 4096 || num_tiles < 0 || num_tiles == INT32_MAX)
    return BSG_ERR_SHAPE;
  if (!counts || !expert_offsets || !tile_offsets || (num_tiles > 0 && !expert_ids))
    return BSG_ERR_NULL;
  if (!aligned(counts, 4) || !aligned(expert_offsets, 4) || !aligned(tile_offsets, 4) ||
      (expert_ids && !aligned(expert_ids, 4)))
    return BSG_ERR_ALIGN;
  if (int st = check_device()) return st;
  hipError_t err = bsg::launch_build_tiles(counts, num_experts, num_tiles, padded ? 1 : 0,
                                           expert_offsets, tile_offsets, expert_ids,
                                           static_cast<hipStream_t>(stream));
  return err == hipSuccess ? BSG_OK : BSG_ERR_LAUNCH;
}

extern "C" int bsgemm_route_counts(const int32_t* topk_ids, int32_t num_picks, int32_t num_experts,
                                   int32_t* counts, void* stream) {
  if (num_experts < 1 || num_experts > 4096 || num_picks < 0) return BSG_ERR_SHAPE;
  if ((num_picks > 0 && !topk_ids) || !counts) return BSG_ERR_NULL;
  if ((topk_ids && !aligned(topk_ids, 4)) || !aligned(counts, 4)) return BSG_ERR_ALIGN;
  if (int st = check_device()) return st;
  hipError_t err = bsg::launch_route_counts(topk_ids, num_picks, num_experts, counts,
                                            static_cast<hipStream_t>(stream));
  return err == hipSuccess ? BSG_OK : BSG_ERR_LAUNCH;
}

extern "C" int bsgemm_quantize_permute(const void* x, uint32_t x_dtype, const int32_t* topk_ids,
                                       int32_t tokens, int32_t top_k, int32_t K, int32_t num_experts,
                                       const int32_t* expert_offsets, int32_t M, int32_t* dest,
                                       void* qa, float* a_scales, void* stream) {
  if (x_dtype != BSG_OUT_F32 && x_dtype != BSG_OUT_BF16) return BSG_ERR_FMT;
  if (tokens < 0 || top_k < 1 || K <= 0 || K % 128 || M < 0 || num_experts < 1 ||
      num_experts > 4096 || (long long)tokens * top_k > INT32_MAX)
    return BSG_ERR_SHAPE;
  if (!expert_offsets || (M > 0 && (!qa || !a_scales)) ||
      (tokens > 0 && (!x || !topk_ids || !dest)))
    return BSG_ERR_NULL;
  if ((x && !aligned(x, 16)) || (qa && !aligned(qa, 16)) || (a_scales && !aligned(a_scales, 4)) ||
      (topk_ids && !aligned(topk_ids, 4)) || (dest && !aligned(dest, 4)) || !aligned(expert_offsets, 4))
    return BSG_ERR_ALIGN;
  if (int st = check_device()) return st;
  hipError_t err = bsg::launch_quantize_permute(x, x_dtype == BSG_OUT_F32 ? 1 : 0, topk_ids, tokens, top_k,
                                                K, num_experts, expert_offsets, M, dest,
                                                static_cast<uint8_t*>(qa), a_scales,
                                                static_cast<hipStream_t>(stream));
  return err == hipSuccess ? BSG_OK : BSG_ERR_LAUNCH;
}

namespace {

// Validation and argument set-up shared by the bsgemm_grouped entry points. Returns BSG_OK with
// *noop set when there is nothing to launch.
int grouped_args(const void* A, const void* a_scales, const void* B, const void* b_scales,
                 const int32_t* expert_ids, const int32_t* tile_offsets, int32_t num_tiles, void* C,
                 int32_t M, int32_t N, int32_t K, int32_t num_experts, uint32_t fmt, bsg::GemmArgs* args,
                 bool* noop) {
  *noop = false;
  const unsigned fa = fmt & 0xF, fb = (fmt >> 4) & 0xF, sk = (fmt >> 8) & 0xF, out = (fmt >> 12) & 0xF;
  const unsigned hint = fmt >> 16;
  if (hint > 1 || out < BSG_OUT_F32 || out > BSG_OUT_F16) return BSG_ERR_FMT;
  if (hint && sk != BSG_SCALE_BLOCKWISE) return BSG_ERR_FMT;
  if (sk == BSG_SCALE_BLOCKWISE) {
    if (fa != BSG_ELEM_E4M3 || fb != BSG_ELEM_E4M3) return BSG_ERR_FMT;
  } else if (sk == BSG_SCALE_MX) {
    if ((fa != BSG_ELEM_E4M3 && fa != BSG_ELEM_E2M1) || (fb != BSG_ELEM_E4M3 && fb != BSG_ELEM_E2M1))
      return BSG_ERR_FMT;
  } else if (sk == BSG_SCALE_NV) {
    if (fa != BSG_ELEM_E2M1 || fb != BSG_ELEM_E2M1) return BSG_ERR_FMT;
  } else {
    return BSG_ERR_FMT;
  }
  if (M < 0 || N <= 0 || K <= 0 || N % 128 || K % 128 || num_experts < 1 || num_tiles < 0)
    return BSG_ERR_SHAPE;
  if (sk == BSG_SCALE_NV && K % 256) return BSG_ERR_SHAPE;
  const bool dense = expert_ids == nullptr && tile_offsets == nullptr;
  if (!dense && (expert_ids == nullptr || tile_offsets == nullptr)) return BSG_ERR_NULL;
  if (!A || !a_scales || !B || !b_scales || !C) return BSG_ERR_NULL;
  const uintptr_t scale_align = sk == BSG_SCALE_NV ? 16 : 4;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(a_scales, scale_align) ||
      !aligned(b_scales, scale_align) || (!dense && (!aligned(expert_ids, 4) || !aligned(tile_offsets, 4))))
    return BSG_ERR_ALIGN;
  if (M == 0 || (!dense && num_tiles == 0)) {
    *noop = true;
    return BSG_OK;
  }
  int num_cus = 0;
  if (int st = check_device(&num_cus)) return st;

  args->A = A;
  args->a_scales = a_scales;
  args->B = B;
  args->b_scales = b_scales;
  args->expert_ids = dense ? nullptr : expert_ids;
  args->tile_offsets = dense ? nullptr : tile_offsets;
  args->C = C;
  args->M = M;
  args->N = N;
  args->K = K;
  args->num_experts = dense ? 1 : num_experts;
  args->num_tiles = dense ? (M + 127) / 128 : num_tiles;
  args->num_cus = num_cus;
  return BSG_OK;
}

// The launch for a validated call: blockwise with the split schedule when a workspace is given.
int grouped_launch(const bsg::GemmArgs& args, uint32_t fmt, void* workspace, size_t workspace_bytes,
                   hipStream_t s) {
  const unsigned fa = fmt & 0xF, fb = (fmt >> 4) & 0xF, sk = (fmt >> 8) & 0xF, out = (fmt >> 12) & 0xF;
  const unsigned hint = fmt >> 16;
  hipError_t err;
  if (sk == BSG_SCALE_BLOCKWISE) {
    if (hint)
      err = bsg::launch_blockwise_fp8_small_m(args, static_cast<int>(out), s);
    else if (workspace)
      err = bsg::launch_blockwise_fp8_split(args, static_cast<int>(out), workspace, workspace_bytes, s);
    else
      err = bsg::launch_blockwise_fp8(args, static_cast<int>(out), s);
  } else if (sk == BSG_SCALE_MX) {
    err = bsg::launch_mx(args, static_cast<int>(fa), static_cast<int>(fb), static_cast<int>(out), s);
  } else {
    err = bsg::launch_nvfp4(args, static_cast<int>(out), s);
  }
  return err == hipSuccess ? BSG_OK : BSG_ERR_LAUNCH;
}

}  // namespace

extern "C" int bsgemm_grouped(const void* A, const void* a_scales, const void* B,
                              const void* b_scales, const int32_t* expert_ids,
                              const int32_t* tile_offsets, int32_t num_tiles, void* C, int32_t M,
                              int32_t N, int32_t K, int32_t num_experts, uint32_t fmt,
                              void* stream) {
  bsg::GemmArgs args;
  bool noop;
  if (int st = grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, num_tiles, C, M, N, K,
                            num_experts, fmt, &args, &noop))
    return st;
  if (noop) return BSG_OK;
  return grouped_launch(args, fmt, nullptr, 0, static_cast<hipStream_t>(stream));
}

extern "C" int bsgemm_grouped_workspace_size(size_t* bytes) {
  if (!bytes) return BSG_ERR_NULL;
  int num_cus = 0;
  if (int st = check_device(&num_cus)) return st;
  *bytes = bsg::blockwise_fp8_workspace_bytes(num_cus);
  return BSG_OK;
}

extern "C" int bsgemm_grouped_ws(const void* A, const void* a_scales, const void* B,
                                 const void* b_scales, const int32_t* expert_ids,
                                 const int32_t* tile_offsets, int32_t num_tiles, void* C, int32_t M,
                                 int32_t N, int32_t K, int32_t num_experts, uint32_t fmt,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  bsg::GemmArgs args;
  bool noop;
  if (int st = grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, num_tiles, C, M, N, K,
                            num_experts, fmt, &args, &noop))
    return st;
  if (!workspace) return BSG_ERR_NULL;
  if (!aligned(workspace, 256)) return BSG_ERR_ALIGN;
  if (noop) return BSG_OK;
  if (workspace_bytes < bsg::blockwise_fp8_workspace_bytes(args.num_cus)) return BSG_ERR_SHAPE;
  return grouped_launch(args, fmt, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" int bsgemm_grouped_noalloc(const void* A, const void* a_scales, const void* B,
                                      const void* b_scales, const int32_t* expert_ids,
                                      const int32_t* tile_offsets, int32_t num_tiles, void* C,
                                      int32_t M, int32_t N, int32_t K, int32_t num_experts,
                                      uint32_t fmt, void* stream) {
  bsg::GemmArgs args;
  bool noop;
  if (int st = grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, num_tiles, C, M, N, K,
                            num_experts, fmt, &args, &noop))
    return st;
  if (noop) return BSG_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return BSG_ERR_DEVICE;
  }
  void* ws = scratch_ptr(dev);
  if (!ws) return BSG_ERR_DEVICE;
  return grouped_launch(args, fmt, ws, kScratchBytes, static_cast<hipStream_t>(stream));
}
