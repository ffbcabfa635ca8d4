/*
 * bsgemm.h - C ABI of the MI355X (gfx950) grouped block-scaled low-precision GEMM.
 *
 * The operation is the grouped, blockwise-FP8 MoE matmul whose per-K-block promote step is
 * described on the Modular MAX page "promote_accumulators"
 * (kernels/linalg/grouped_matmul_sm100_blockwise_fp8; description paragraph and section
 * Args), with the per-K-iteration cadence of the Modular MAX page "EpilogueWarpContext"
 * (method per_k_stage), plus the MX variant of the Triton Gluon page "Overlapping
 * Accumulator Block-Scaled Matrix Multiplication" (e8m0 scale per 32 K-elements, applied
 * inside the matrix instruction; reference result A_ref @ B_ref^T in its make_problem).
 *
 * General rules for every entry point:
 *  - Pointers marked DEVICE are device (HBM) pointers owned by the caller. The library
 *    never allocates, frees or retains them. Pointers marked HOST are host pointers.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL means
 *    the null stream) on the current HIP device. Calls return after enqueueing.
 *  - Return value: BSG_OK (0) or a negative bsg_status. Arguments are validated on the host
 *    before anything is enqueued; on any error nothing is enqueued and outputs are untouched.
 *  - Thread-safe: no global mutable state apart from a per-device property cache.
 *  - Device-side contents (tile map, counts) cannot be checked on the host. The kernels clamp
 *    them instead: a tile whose expert id is outside [0, num_experts) is skipped, rows are
 *    clamped into [0, M), and negative counts count as zero. Such input gives unspecified
 *    (but in-bounds) results.
 */
#ifndef BSGEMM_H
#define BSGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSG_OK = 0,
  BSG_ERR_NULL = -1,    /* a required pointer is NULL                                   */
  BSG_ERR_SHAPE = -2,   /* a size is negative, too large, or not a multiple it must be  */
  BSG_ERR_ALIGN = -3,   /* a pointer is not aligned as documented                      */
  BSG_ERR_FMT = -4,     /* unsupported fmt combination                                 */
  BSG_ERR_DEVICE = -5,  /* no HIP device, or the current device is not gfx950          */
  BSG_ERR_LAUNCH = -6   /* the HIP runtime rejected a kernel launch                    */
} bsg_status;

/* ---- fmt: element formats, scale kind and output type, packed into one word ------------ */
#define BSG_ELEM_E4M3 1u   /* OCP e4m3fn, one byte per element                            */
#define BSG_ELEM_E2M1 2u   /* OCP e2m1, two per byte along K, even K index in low nibble  */
#define BSG_SCALE_BLOCKWISE 1u /* fp32: A per row per 128 K; B per 128 (N) x 128 (K) block */
#define BSG_SCALE_MX 2u        /* e8m0 (uint8, 2^(x-127)): one per row per 32 K, A and B   */
#define BSG_SCALE_NV 3u        /* nvfp4: e4m3fn (uint8) scale per row per 16 K, A and B    */
#define BSG_OUT_F32 1u
#define BSG_OUT_BF16 2u
#define BSG_OUT_F16 3u
#define BSG_FMT(a_elem, b_elem, scale, out) \
  ((uint32_t)(a_elem) | ((uint32_t)(b_elem) << 4) | ((uint32_t)(scale) << 8) | ((uint32_t)(out) << 12))
/* Schedule hint (OR into fmt; blockwise only): M-tiles hold few rows (decode-sized expert
 * groups). Each work item is then one M-tile x 256 columns, and the matrix work stops at the
 * tile's last row of 16-row fragments, instead of a 256 x 256 block tile. Same results, bit for
 * bit (same instruction, operand roles and promotion order). Only the packed tile layout
 * (bsgemm_build_tiles with padded == 0) has tiles of fewer than 128 rows: with the padded layout
 * every tile spans 128 rows (padding included), so no fragment is skipped and the hint only
 * changes the work item's shape. */
#define BSG_SCHED_SMALL_M (1u << 16)

/*
 * bsgemm_build_tiles - token-to-expert tile map (the scheduler build).
 *
 * Passage: "promote_accumulators", section Args, argument expert_ids (maps a group of rows
 * to its expert in B) and argument scheduler (tracks the current group and work tile).
 *
 * Rows of A are grouped by expert in ascending expert order. From the per-expert row counts
 * this writes, with T = num_tiles:
 *   expert_offsets[e]  first row of expert e's group; expert_offsets[E] = rows the layout needs
 *   tile_offsets[t]    first row of M-tile t (t in [0, T]); tile t owns
 *                      min(128, max(0, tile_offsets[t+1] - tile_offsets[t])) rows
 *   expert_ids[t]      expert of M-tile t, or -1 for tiles past the last expert's rows
 * padded != 0: each group starts at a multiple of 128 rows, tile_offsets[t] = 128 t, and tiles
 *   include the group's padding rows.
 * padded == 0: groups are packed back to back; each group's last tile is ragged; tiles past
 *   the last one start at expert_offsets[E].
 * If the layout needs more than T tiles, the extra tiles are dropped (expert_offsets[E] still
 * reports the rows needed, so the caller can detect it).
 *
 *   counts          DEVICE int32[num_experts], row count per expert (>= 0)
 *   num_experts     1 .. 4096
 *   num_tiles       >= 0
 *   expert_offsets  DEVICE int32[num_experts + 1] (output)
 *   tile_offsets    DEVICE int32[num_tiles + 1]   (output)
 *   expert_ids      DEVICE int32[num_tiles]       (output; may be NULL iff num_tiles == 0)
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_ALIGN (int32 alignment), BSG_ERR_DEVICE,
 * BSG_ERR_LAUNCH.
 */
int bsgemm_build_tiles(const int32_t* counts, int32_t num_experts, int32_t num_tiles,
                       int32_t padded, int32_t* expert_offsets, int32_t* tile_offsets,
                       int32_t* expert_ids, void* stream);

/*
 * bsgemm_grouped - grouped block-scaled GEMM  C[rows of tile t] = A[rows] * B[e]^T, e = expert_ids[t].
 *
 * Blockwise (scale kind BSG_SCALE_BLOCKWISE; passage: "promote_accumulators", description
 * paragraph, and Args b_scales / b_scales_n / k_iter / expert_ids / problem_shape):
 *   for every K block kb of 128:  P = sum_{k in kb} qa[m,k] * qb[e,n,k]   (fp32, fresh each block)
 *                                 acc[m,n] += P * (a_scales[m,kb] * b_scales[e, n/128, kb])
 *   C[m,n] = acc[m,n] converted to the output type (round to nearest even).
 * MX (BSG_SCALE_MX; passage: Gluon page, random_quantized_tensor / async_mma_scaled_impl):
 *   C[m,n] = sum_k (qa[m,k] 2^(sa[m,k/32]-127)) (qb[e,n,k] 2^(sb[e,n,k/32]-127)), scales
 *   applied by the gfx950 scaled matrix instruction, fp32 accumulation.
 * nvfp4 (BSG_SCALE_NV; passage: Gluon page, random_quantized_tensor for "nvfp4", VEC_SIZE 16,
 *   scales converted to float8_e4m3fn):
 *   C[m,n] = sum_k (e2m1(qa[m,k]) e4m3(sa[m,k/16])) (e2m1(qb[e,n,k]) e4m3(sb[e,n,k/16])), each
 *   scaled element formed exactly in f16, fp32 accumulation.
 *
 * Layouts (all row-major, contiguous):
 *   A          DEVICE [M, K] e4m3 bytes, or [M, K/2] packed e2m1. 16-byte aligned.
 *   a_scales   blockwise: DEVICE float[M, K/128];  MX: DEVICE uint8[M, K/32]. 4-byte aligned.
 *              nvfp4: DEVICE uint8[M, K/16] e4m3fn codes, 16-byte aligned.
 *   B          DEVICE [num_experts, N, K] e4m3 (or [num_experts, N, K/2] e2m1): K contiguous,
 *              i.e. each expert's B is stored N-major ("NT" GEMM). 16-byte aligned.
 *   b_scales   blockwise: DEVICE float[num_experts, N/128, K/128];
 *              MX: DEVICE uint8[num_experts, N, K/32]. 4-byte aligned.
 *              nvfp4: DEVICE uint8[num_experts, N, K/16] e4m3fn codes, 16-byte aligned.
 *   expert_ids DEVICE int32[num_tiles] and tile_offsets DEVICE int32[num_tiles + 1], as written
 *              by bsgemm_build_tiles (either layout). Both NULL: one dense group, expert 0,
 *              tiles of 128 rows, num_tiles ignored (M need not be a multiple of 128).
 *   C          DEVICE [M, N] float / bf16 / fp16. 16-byte aligned. Rows of skipped tiles and
 *              rows no tile covers are not written.
 * Sizes: M >= 0 (M = 0 is a no-op), N > 0 and K > 0, both multiples of 128; num_experts >= 1;
 *   num_tiles >= 0.
 * Supported fmt: blockwise with A = B = e4m3, any output type (optionally | BSG_SCHED_SMALL_M);
 *   MX with A, B in {e4m3, e2m1}, any output type;
 *   nvfp4 with A = B = e2m1 and K a multiple of 256 (else BSG_ERR_SHAPE), any output type.
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_ALIGN, BSG_ERR_FMT, BSG_ERR_DEVICE,
 *   BSG_ERR_LAUNCH.
 */
/*
 * Arguments beyond the problem statement's list. The operation is named with the arguments
 * (A, a_scales, B, b_scales, expert_ids, tile_offsets, C, M, N, K, fmt, stream). Two more are
 * taken here: num_tiles, the length of expert_ids (a ragged, unpadded layout has a tile count
 * that M does not determine, and the kernels never read past it), and num_experts, the leading
 * dimension of B and b_scales ("promote_accumulators", Args: b_scales is shaped
 * [num_experts, N // BN, K // BK]), so that an out-of-range expert id is skipped instead of
 * addressing past B. Neither changes the result for a valid tile map.
 */
int bsgemm_grouped(const void* A, const void* a_scales, const void* B, const void* b_scales,
                   const int32_t* expert_ids, const int32_t* tile_offsets, int32_t num_tiles,
                   void* C, int32_t M, int32_t N, int32_t K, int32_t num_experts, uint32_t fmt,
                   void* stream);

/*
 * bsgemm_grouped_workspace_size - bytes of workspace bsgemm_grouped_ws needs on the current device.
 *
 *   bytes   HOST size_t* (output): 4 KiB of flags plus one 256 x 256 fp32 tile per workgroup of
 *           the split schedule (one per compute unit, rounded down to a multiple of 8: 64 MiB + 4 KiB
 *           on a 256-CU MI355X)
 * Errors: BSG_ERR_NULL, BSG_ERR_DEVICE.
 */
int bsgemm_grouped_workspace_size(size_t* bytes);

/*
 * bsgemm_grouped_ws - bsgemm_grouped with a workspace for a split-K schedule of small problems.
 *
 * Same operation, arguments and results as bsgemm_grouped (up to the rounding order of fp32 sums:
 * outputs are within the same tolerance, not bit-identical). bsgemm_grouped runs one 256 x 256
 * work item per workgroup, so a problem with fewer items than compute units leaves units idle
 * (a 256 x 2048 x 16384 GEMM has 8 items for 256 units). With a workspace, such blockwise calls
 * cut each item along K into 2-16 equal ranges of at least 8 K blocks (as many as the grid
 * holds) that run side by side: each range accumulates its K blocks as described under
 * bsgemm_grouped into an fp32 partial tile, and the item's result is the sum of its ranges'
 * partials (each range sums and stores a slice of the tile). Blockwise problems with at least as
 * many items as compute units run whole items as bsgemm_grouped does, bit for bit, with two
 * exceptions that use the workspace's first 4 KiB as counters and flags (cleared on the stream
 * before the launch):
 *  - when K is at least 5120 (40 K blocks), the workgroups take the items of each XCD from a
 *    counter instead of a fixed sequence, which keeps the items in flight on an XCD close
 *    together in the work order (same per-item arithmetic: still bit for bit);
 *  - with fewer than 4 items per compute unit, the items of the last, partial round (items modulo
 *    the grid) are cut along K into 2-16 ranges of at least 4 K blocks, which the workgroups that
 *    run out of whole items first take from a counter, summed as above; outputs of those items
 *    are within the tolerance, not bit-identical to bsgemm_grouped, and the same on every call.
 * Formats other than blockwise and the small-M hint run exactly as bsgemm_grouped and leave the
 * workspace untouched.
 *
 *   workspace        DEVICE, 256-byte aligned, at least bsgemm_grouped_workspace_size bytes,
 *                    owned by the caller; no initial contents are required (what a launch
 *                    uses of it is cleared on the stream before the launch). Its int32 word 1023 is
 *                    an error word: nonzero after a call if a range ever stopped waiting for the
 *                    other ranges of its item (not expected while the call has the GPU's compute
 *                    units to itself: the ranges wait for ranges that running workgroups have
 *                    taken; that item's output is then wrong).
 *   workspace_bytes  its size
 * Calls that share a workspace must be ordered (one stream, or synchronised): concurrent calls
 * on one workspace race.
 * Errors: as bsgemm_grouped, plus BSG_ERR_NULL (workspace NULL), BSG_ERR_ALIGN, BSG_ERR_SHAPE
 * (workspace too small).
 */
int bsgemm_grouped_ws(const void* A, const void* a_scales, const void* B, const void* b_scales,
                      const int32_t* expert_ids, const int32_t* tile_offsets, int32_t num_tiles,
                      void* C, int32_t M, int32_t N, int32_t K, int32_t num_experts, uint32_t fmt,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsgemm_grouped_noalloc - bsgemm_grouped_ws without a workspace argument, allocating nothing.
 *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same operation, arguments, results and errors as
 * bsgemm_grouped; its split-K schedule for small problems (see bsgemm_grouped_ws) uses a scratch
 * array the library holds on each device it runs on, for the life of the process: 16 MiB + 4 KiB,
 * room for 64 partial tiles. Where bsgemm_grouped_ws would cut the items into more ranges than
 * 64 tiles, fewer ranges are used, so no call needs more scratch than the array holds and none
 * is rejected for it (results are within the same tolerance). What a launch uses of the scratch
 * (the split schedule's flags, the work-order counters) is cleared on the stream before it.
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one GPU (different streams
 * or host threads without ordering) race and give wrong results. No hipMalloc, hipFree or other
 * allocating call is made.
 */
int bsgemm_grouped_noalloc(const void* A, const void* a_scales, const void* B, const void* b_scales,
                           const int32_t* expert_ids, const int32_t* tile_offsets, int32_t num_tiles,
                           void* C, int32_t M, int32_t N, int32_t K, int32_t num_experts, uint32_t fmt,
                           void* stream);

/*
 * bsgemm_route_counts - picks per expert: the row counts of the grouped A.
 *
 * Passage: "promote_accumulators", section Args, argument expert_ids (each group of A's rows
 * belongs to one expert) - the counts that bsgemm_build_tiles turns into the group layout.
 *
 *   topk_ids    DEVICE int32[num_picks]: expert of each pick, usually [tokens, top_k]
 *               row-major. Ids outside [0, num_experts) are not counted.
 *   num_picks   >= 0
 *   num_experts 1 .. 4096
 *   counts      DEVICE int32[num_experts] (output; overwritten)
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_ALIGN (int32 alignment), BSG_ERR_DEVICE,
 * BSG_ERR_LAUNCH.
 */
int bsgemm_route_counts(const int32_t* topk_ids, int32_t num_picks, int32_t num_experts,
                        int32_t* counts, void* stream);

/*
 * bsgemm_quantize_permute - token activations and top-k picks -> the grouped GEMM's A operand.
 *
 * Passage: "promote_accumulators", section Args (A's rows grouped by expert through
 * expert_ids; an fp32 scale per row per 128 K-elements, the 1x128 block scaling of the FP8
 * operands). The pages do not order rows inside a group; here expert e's picks fill rows
 * expert_offsets[e], expert_offsets[e] + 1, ... in pick order (token-major), which makes the
 * layout unique.
 *
 *   dest[t, j]   = A row of pick (t, j), or -1 if its id is outside [0, num_experts) or the
 *                  row would be >= M
 *   per token t and 128-block b of x[t]:  s = amax / 448 (1 if amax = 0),
 *                  q = round-to-nearest-even e4m3fn of clamp(x / s, -448, 448), both divisions
 *                  in fp32; qa[dest[t, j], block b] = q and a_scales[dest[t, j], b] = s
 *   rows expert_offsets[e] + count_e .. expert_offsets[e + 1] - 1 (below M): zero codes,
 *                  scale 1 (the group's padding); all other rows of qa / a_scales untouched
 *
 *   x              DEVICE [tokens, K] fp32 or bf16 (x_dtype BSG_OUT_F32 / BSG_OUT_BF16),
 *                  finite values. 16-byte aligned.
 *   topk_ids       DEVICE int32[tokens, top_k]
 *   tokens >= 0, top_k >= 1, K > 0 a multiple of 128, num_experts 1 .. 4096
 *   expert_offsets DEVICE int32[num_experts + 1], as written by bsgemm_build_tiles from
 *                  bsgemm_route_counts' counts (padded: each group a multiple of 128 rows)
 *   M              rows of qa / a_scales (>= 0)
 *   dest           DEVICE int32[tokens, top_k] (output)
 *   qa             DEVICE uint8[M, K] e4m3fn codes (output), 16-byte aligned
 *   a_scales       DEVICE float[M, K/128] (output)
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_ALIGN, BSG_ERR_FMT (x_dtype), BSG_ERR_DEVICE,
 * BSG_ERR_LAUNCH.
 */
int bsgemm_quantize_permute(const void* x, uint32_t x_dtype, const int32_t* topk_ids,
                            int32_t tokens, int32_t top_k, int32_t K, int32_t num_experts,
                            const int32_t* expert_offsets, int32_t M, int32_t* dest, void* qa,
                            float* a_scales, void* stream);

/* Static, human-readable text for a bsg_status value (never NULL). */
const char* bsgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BSGEMM_H */
