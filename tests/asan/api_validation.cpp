// Host-side checks of the C-ABI validation layer (bsgemm_api.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host part only and run without a GPU: every entry point is
// called with NULL, misaligned, out-of-range and well-formed arguments. The kernels' launchers
// are replaced by stubs here (nothing reaches them without a device); a well-formed call must
// come back with BSG_ERR_DEVICE. Exit status 0 when every return code is the documented one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "bsgemm.h"
#include "launch.h"

namespace bsg {
// Launchers: never reached without a device (the device check comes first).
hipError_t launch_blockwise_fp8(const GemmArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_blockwise_fp8_split(const GemmArgs&, int, void*, size_t, hipStream_t) { return hipErrorInvalidValue; }
size_t blockwise_fp8_workspace_bytes(int num_cus) { return 4096 + (size_t)num_cus * 256 * 256 * 4; }
hipError_t launch_blockwise_fp8_small_m(const GemmArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mx(const GemmArgs&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_nvfp4(const GemmArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_route_counts(const int32_t*, int, int, int32_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quantize_permute(const void*, int, const int32_t*, int, int, int, int, const int32_t*, int,
                                   int32_t*, uint8_t*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_build_tiles(const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace bsg

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %-48s got %d (%s), want %d (%s)\n", what, got, bsgemm_status_string(got), want,
                bsgemm_status_string(want));
    failures++;
  }
}

int main() {
  alignas(256) static unsigned char buf[1 << 16];
  unsigned char* u = buf + 1;                              // misaligned for every rule
  const int32_t* i32 = reinterpret_cast<const int32_t*>(buf);
  int32_t* o32 = reinterpret_cast<int32_t*>(buf + 4096);
  const uint32_t bw = BSG_FMT(BSG_ELEM_E4M3, BSG_ELEM_E4M3, BSG_SCALE_BLOCKWISE, BSG_OUT_BF16);
  const uint32_t mx = BSG_FMT(BSG_ELEM_E2M1, BSG_ELEM_E4M3, BSG_SCALE_MX, BSG_OUT_F16);
  const uint32_t nv = BSG_FMT(BSG_ELEM_E2M1, BSG_ELEM_E2M1, BSG_SCALE_NV, BSG_OUT_F32);

  // status strings: every code, and an unknown one, give static text
  for (int s = -8; s <= 1; s++) expect("status string non-empty", std::strlen(bsgemm_status_string(s)) > 0, 1);

  // bsgemm_grouped (dense and grouped), every rule
  expect("grouped: A NULL", bsgemm_grouped(nullptr, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_NULL);
  expect("grouped: C NULL", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, nullptr, 128, 256, 512, 1, bw, nullptr), BSG_ERR_NULL);
  expect("grouped: one of the tile map NULL", bsgemm_grouped(buf, buf, buf, buf, i32, nullptr, 1, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_NULL);
  expect("grouped: A misaligned", bsgemm_grouped(u, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_ALIGN);
  expect("grouped: C misaligned", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, u, 128, 256, 512, 1, bw, nullptr), BSG_ERR_ALIGN);
  expect("grouped: scales misaligned", bsgemm_grouped(buf, u, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_ALIGN);
  expect("grouped: N not a multiple of 128", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 200, 512, 1, bw, nullptr), BSG_ERR_SHAPE);
  expect("grouped: K not a multiple of 128", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 500, 1, bw, nullptr), BSG_ERR_SHAPE);
  expect("grouped: M negative", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, -1, 256, 512, 1, bw, nullptr), BSG_ERR_SHAPE);
  expect("grouped: num_tiles negative", bsgemm_grouped(buf, buf, buf, buf, i32, i32, -3, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_SHAPE);
  expect("grouped: no experts", bsgemm_grouped(buf, buf, buf, buf, i32, i32, 1, buf, 128, 256, 512, 0, bw, nullptr), BSG_ERR_SHAPE);
  expect("grouped: nvfp4 with K % 256", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 384, 1, nv, nullptr), BSG_ERR_SHAPE);
  expect("grouped: unknown scale kind", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, BSG_FMT(1u, 1u, 7u, 2u), nullptr), BSG_ERR_FMT);
  expect("grouped: blockwise with e2m1", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, BSG_FMT(2u, 1u, 1u, 2u), nullptr), BSG_ERR_FMT);
  expect("grouped: bad output type", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, BSG_FMT(1u, 1u, 1u, 9u), nullptr), BSG_ERR_FMT);
  expect("grouped: small-M hint on MX", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, mx | BSG_SCHED_SMALL_M, nullptr), BSG_ERR_FMT);
  expect("grouped: M = 0 is a no-op", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 0, 256, 512, 1, bw, nullptr), BSG_OK);
  expect("grouped: no tiles is a no-op", bsgemm_grouped(buf, buf, buf, buf, i32, i32, 0, buf, 128, 256, 512, 4, bw, nullptr), BSG_OK);
  expect("grouped: well formed, no device", bsgemm_grouped(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_DEVICE);
  expect("grouped: MX well formed, no device", bsgemm_grouped(buf, buf, buf, buf, i32, i32, 2, buf, 256, 256, 512, 3, mx, nullptr), BSG_ERR_DEVICE);

  // bsgemm_grouped_workspace_size / _ws / _noalloc
  expect("workspace size: NULL", bsgemm_grouped_workspace_size(nullptr), BSG_ERR_NULL);
  size_t bytes = 0;
  expect("workspace size: no device", bsgemm_grouped_workspace_size(&bytes), BSG_ERR_DEVICE);
  expect("ws: workspace NULL", bsgemm_grouped_ws(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 0, 256, 512, 1, bw, nullptr, 0, nullptr), BSG_ERR_NULL);
  expect("ws: workspace misaligned", bsgemm_grouped_ws(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 0, 256, 512, 1, bw, buf + 16, 4096, nullptr), BSG_ERR_ALIGN);
  expect("ws: argument error first", bsgemm_grouped_ws(nullptr, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, nullptr, 0, nullptr), BSG_ERR_NULL);
  expect("ws: well formed, no device", bsgemm_grouped_ws(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, buf, sizeof buf, nullptr), BSG_ERR_DEVICE);
  expect("noalloc: argument error", bsgemm_grouped_noalloc(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 255, 512, 1, bw, nullptr), BSG_ERR_SHAPE);
  expect("noalloc: well formed, no device", bsgemm_grouped_noalloc(buf, buf, buf, buf, nullptr, nullptr, 0, buf, 128, 256, 512, 1, bw, nullptr), BSG_ERR_DEVICE);

  // bsgemm_build_tiles
  expect("tiles: no experts", bsgemm_build_tiles(i32, 0, 4, 1, o32, o32, o32, nullptr), BSG_ERR_SHAPE);
  expect("tiles: too many experts", bsgemm_build_tiles(i32, 4097, 4, 1, o32, o32, o32, nullptr), BSG_ERR_SHAPE);
  expect("tiles: num_tiles INT32_MAX", bsgemm_build_tiles(i32, 4, INT32_MAX, 1, o32, o32, o32, nullptr), BSG_ERR_SHAPE);
  expect("tiles: counts NULL", bsgemm_build_tiles(nullptr, 4, 4, 1, o32, o32, o32, nullptr), BSG_ERR_NULL);
  expect("tiles: expert_ids NULL with tiles", bsgemm_build_tiles(i32, 4, 4, 1, o32, o32, nullptr, nullptr), BSG_ERR_NULL);
  expect("tiles: misaligned", bsgemm_build_tiles(i32, 4, 4, 1, reinterpret_cast<int32_t*>(u), o32, o32, nullptr), BSG_ERR_ALIGN);
  expect("tiles: well formed, no device", bsgemm_build_tiles(i32, 4, 0, 0, o32, o32, nullptr, nullptr), BSG_ERR_DEVICE);

  // bsgemm_route_counts
  expect("route: negative picks", bsgemm_route_counts(i32, -1, 4, o32, nullptr), BSG_ERR_SHAPE);
  expect("route: counts NULL", bsgemm_route_counts(i32, 8, 4, nullptr, nullptr), BSG_ERR_NULL);
  expect("route: ids NULL with picks", bsgemm_route_counts(nullptr, 8, 4, o32, nullptr), BSG_ERR_NULL);
  expect("route: misaligned", bsgemm_route_counts(reinterpret_cast<const int32_t*>(u), 8, 4, o32, nullptr), BSG_ERR_ALIGN);
  expect("route: well formed, no device", bsgemm_route_counts(nullptr, 0, 4, o32, nullptr), BSG_ERR_DEVICE);

  // bsgemm_quantize_permute
  float* sc = reinterpret_cast<float*>(buf + 8192);
  expect("permute: bad x dtype", bsgemm_quantize_permute(buf, 3u, i32, 4, 2, 256, 4, i32, 16, o32, buf, sc, nullptr), BSG_ERR_FMT);
  expect("permute: K % 128", bsgemm_quantize_permute(buf, BSG_OUT_BF16, i32, 4, 2, 200, 4, i32, 16, o32, buf, sc, nullptr), BSG_ERR_SHAPE);
  expect("permute: tokens x top_k overflow", bsgemm_quantize_permute(buf, BSG_OUT_BF16, i32, INT32_MAX, 2, 256, 4, i32, 16, o32, buf, sc, nullptr), BSG_ERR_SHAPE);
  expect("permute: x NULL", bsgemm_quantize_permute(nullptr, BSG_OUT_BF16, i32, 4, 2, 256, 4, i32, 16, o32, buf, sc, nullptr), BSG_ERR_NULL);
  expect("permute: qa misaligned", bsgemm_quantize_permute(buf, BSG_OUT_F32, i32, 4, 2, 256, 4, i32, 16, o32, u, sc, nullptr), BSG_ERR_ALIGN);
  expect("permute: well formed, no device", bsgemm_quantize_permute(buf, BSG_OUT_F32, i32, 4, 2, 256, 4, i32, 16, o32, buf, sc, nullptr), BSG_ERR_DEVICE);

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
