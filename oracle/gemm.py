"""fp64 CPU oracle for the grouped block-scaled GEMM (test infrastructure only).

Problem statement (Modular MAX page "promote_accumulators",
grouped_matmul_sm100_blockwise_fp8; description paragraph and section Args):
a grouped GEMM whose groups are MoE experts. ``expert_ids`` maps a group of A
rows to the expert whose B it multiplies. For every K iteration the MMA forms
an fp32 partial product of one K block; the promote step fetches the A scale of
each row and the B scale of ``(expert, n block, k_iter)`` from ``b_scales``
shaped ``[num_experts, N // BN, K // BK]``, multiplies them into one scale and
accumulates ``partial * scale`` into the running accumulator. The Modular MAX
page "EpilogueWarpContext" (method ``per_k_stage``) gives the cadence: one
promote per K iteration.

Layout readings used throughout (the pages leave them open):

* A is ``[M, K]`` row-major, rows grouped by expert; ``a_scales`` is
  ``[M, K/128]`` (one scale per row per 128-wide K block).
* B is ``[E, N, K]`` (K contiguous, the Gluon page's ``B`` is ``[N, K]`` and
  enters the MMA permuted); ``b_scales`` is ``[E, N/128, K/128]``.
* Scale blocks are 1x128 for A and 128x128 for B, independent of any kernel tile.
* M-tile ``t`` covers rows ``[tile_offsets[t], tile_offsets[t] + rows_t)`` with
  ``rows_t = clamp(tile_offsets[t+1] - tile_offsets[t], 0, 128)``;
  ``expert_ids[t] < 0`` means the tile is skipped. ``None`` for both means one
  dense group (expert 0, tiles of 128 rows).

MX variant (Triton Gluon page "Overlapping Accumulator Block-Scaled Matrix
Multiplication", ``make_problem`` and ``random_quantized_tensor``): every 32
consecutive K elements of a row of A (of B) share one e8m0 scale, and the
result is ``A_ref @ B_ref.T`` on the dequantised values.

nvfp4 variant (same page, the ``nvfp4`` format of ``random_quantized_tensor``):
e2m1 elements packed two per byte along K, and one ``float8_e4m3fn`` scale per
16 consecutive K elements of a row (``VEC_SIZE = 16``); the result is again
``A_ref @ B_ref.T`` with ``X_ref = e2m1 * scale.repeat_interleave(16)``.
"""

import numpy as np

from .formats import decode_e4m3fn, decode_e8m0, decode_elements

TILE_M = 128      # rows per M-tile of the token-to-expert map
SCALE_BLOCK = 128  # blockwise scale granularity along N (B) and K (A and B)
MX_BLOCK = 32      # K elements per e8m0 scale
NV_BLOCK = 16      # K elements per e4m3 scale (nvfp4)


# --------------------------------------------------------------------------------------
# a1: token-to-expert tile map
# --------------------------------------------------------------------------------------
def tile_map(counts, num_tiles, padded=True):
    """Per-M-tile expert ids and row ranges from per-expert row counts.

    Rows are grouped by expert in ascending expert order (the ``expert_ids``
    argument of "promote_accumulators", section Args, maps a group to its
    expert). ``padded=True``: each expert's group starts at a multiple of 128
    rows and its tiles are whole 128-row tiles (padding rows included).
    ``padded=False``: groups are packed back to back and each group's last tile
    holds only its remaining rows.

    Returns ``(expert_offsets[E+1], tile_offsets[T+1], expert_ids[T])`` as int64
    arrays. ``expert_offsets[e]`` is the first row of expert ``e`` and
    ``expert_offsets[E]`` the total row count the layout needs (which may
    exceed ``128 * T``; tiles past ``T`` are then dropped). Tiles no expert
    reaches get id -1.
    """
    counts = [int(c) for c in counts]
    if any(c < 0 for c in counts):
        raise ValueError("counts must be non-negative")
    E, T = len(counts), int(num_tiles)
    expert_offsets = [0]
    for c in counts:
        size = -(-c // TILE_M) * TILE_M if padded else c
        expert_offsets.append(expert_offsets[-1] + size)

    tile_offsets, expert_ids = [], []
    for e in range(E):
        start, c = expert_offsets[e], counts[e]
        for j in range(-(-c // TILE_M)):
            tile_offsets.append(start + j * TILE_M)
            expert_ids.append(e)
    if padded:
        tile_offsets = [TILE_M * t for t in range(T + 1)]
    else:
        total = expert_offsets[E]
        tile_offsets = (tile_offsets + [total] * (T + 1))[: T + 1]
    expert_ids = (expert_ids + [-1] * T)[:T]
    return (np.array(expert_offsets, np.int64), np.array(tile_offsets, np.int64),
            np.array(expert_ids, np.int64))


def row_experts(expert_ids, tile_offsets, M):
    """Expert of every A row (-1 where no live tile covers the row)."""
    owner = np.full(M, -1, np.int64)
    if expert_ids is None:
        owner[:] = 0
        return owner
    expert_ids = np.asarray(expert_ids, np.int64)
    tile_offsets = np.asarray(tile_offsets, np.int64)
    for t, e in enumerate(expert_ids):
        if e < 0:
            continue
        r0 = int(tile_offsets[t])
        n = int(min(max(int(tile_offsets[t + 1]) - r0, 0), TILE_M))
        r0c, r1c = max(r0, 0), min(r0 + n, M)
        owner[r0c:r1c] = e
    return owner


def _groups(expert_ids, tile_offsets, M, rows):
    """[(expert, row indices)] for the requested rows (all rows if ``rows`` is None)."""
    owner = row_experts(expert_ids, tile_offsets, M)
    sel = np.arange(M) if rows is None else np.unique(np.asarray(rows, np.int64))
    out = []
    for e in np.unique(owner[sel]):
        if e >= 0:
            out.append((int(e), sel[owner[sel] == e]))
    return out, sel


def _expert_b(B, e):
    B = np.asarray(B)
    return B if B.ndim == 2 else B[e]


# --------------------------------------------------------------------------------------
# a3-a6: blockwise FP8 grouped GEMM, K-block by K-block with scale promotion
# --------------------------------------------------------------------------------------
def blockwise_grouped(qa, a_scales, qb, b_scales, expert_ids=None, tile_offsets=None, rows=None):
    """Grouped blockwise-FP8 GEMM, following the promote description step by step.

    ``qa`` uint8 e4m3 ``[M, K]``; ``a_scales`` float32 ``[M, K/128]``;
    ``qb`` uint8 e4m3 ``[E, N, K]`` (or ``[N, K]``); ``b_scales`` float32
    ``[E, N/128, K/128]`` (or ``[N/128, K/128]``).

    For each K block ``kb`` (the ``k_iter`` of "promote_accumulators"):
      1. the partial ``P = qa[rows, kb block] @ qb[e, :, kb block]^T``
         (exact in fp64: every e4m3 product is a multiple of 2**-18 below 2**18);
      2. the scale ``s[m, n] = a_scales[m, kb] * b_scales[e, n // 128, kb]``;
      3. the promotion ``acc += P * s``.

    Returns ``C`` float64 ``[M, N]``; rows no live tile covers (or not in
    ``rows``) are NaN.
    """
    qa = np.asarray(qa, np.uint8)
    M, K = qa.shape
    qb_any = np.asarray(qb)
    N = qb_any.shape[-2]
    if K % SCALE_BLOCK or N % SCALE_BLOCK:
        raise ValueError("N and K must be multiples of 128")
    a_scales = np.asarray(a_scales, np.float64)
    b_scales = np.asarray(b_scales, np.float64)
    C = np.full((M, N), np.nan)
    groups, _ = _groups(expert_ids, tile_offsets, M, rows)
    for e, r in groups:
        a_codes = decode_elements(qa[r], "e4m3")                  # [R, K]
        b_codes = decode_elements(_expert_b(qb, e), "e4m3")       # [N, K]
        bs = b_scales if b_scales.ndim == 2 else b_scales[e]      # [N/128, K/128]
        acc = np.zeros((len(r), N))
        for kb in range(K // SCALE_BLOCK):
            blk = slice(kb * SCALE_BLOCK, (kb + 1) * SCALE_BLOCK)
            partial = a_codes[:, blk] @ b_codes[:, blk].T          # step 1
            s = a_scales[r, kb][:, None] * np.repeat(bs[:, kb], SCALE_BLOCK)[None, :]  # step 2
            acc += partial * s                                     # step 3
        C[r] = acc
    return C


def dequantize_blockwise_a(qa, a_scales):
    """``qa[m, k] * a_scales[m, k // 128]`` in fp64."""
    a = decode_elements(qa, "e4m3")
    return a * np.repeat(np.asarray(a_scales, np.float64), SCALE_BLOCK, axis=-1)


def dequantize_blockwise_b(qb_e, b_scales_e):
    """``qb[n, k] * b_scales[n // 128, k // 128]`` in fp64, for one expert."""
    b = decode_elements(qb_e, "e4m3")
    s = np.asarray(b_scales_e, np.float64)
    return b * np.repeat(np.repeat(s, SCALE_BLOCK, axis=0), SCALE_BLOCK, axis=1)


def dequantize_mx(q, scales, fmt):
    """``decode(q)[r, k] * 2**(scales[r, k // 32] - 127)`` in fp64."""
    v = decode_elements(q, fmt)
    return v * np.repeat(decode_e8m0(scales), MX_BLOCK, axis=-1)


def _grouped_dequant(deq_a, deq_b_of, N, expert_ids, tile_offsets, M, rows, absolute=False):
    C = np.full((M, N), np.nan)
    groups, _ = _groups(expert_ids, tile_offsets, M, rows)
    for e, r in groups:
        a = deq_a(r)
        b = deq_b_of(e)
        if absolute:
            a, b = np.abs(a), np.abs(b)
        C[r] = a @ b.T
    return C


def blockwise_grouped_dequant(qa, a_scales, qb, b_scales, expert_ids=None, tile_offsets=None,
                              rows=None, absolute=False):
    """The same product by its plain definition: ``deq(A)[rows of e] @ deq(B[e])^T``.

    Identical to :func:`blockwise_grouped` up to fp64 rounding, because the
    scale is constant inside each 1x128 (A) and 128x128 (B) block.
    ``absolute=True`` returns ``|deq A| @ |deq B|^T`` instead, the per-element
    magnitude sum used as the error denominator.
    """
    qa = np.asarray(qa, np.uint8)
    M = qa.shape[0]
    N = np.asarray(qb).shape[-2]
    bs = np.asarray(b_scales)

    def deq_b(e):
        return dequantize_blockwise_b(_expert_b(qb, e), bs if bs.ndim == 2 else bs[e])

    return _grouped_dequant(lambda r: dequantize_blockwise_a(qa[r], np.asarray(a_scales)[r]),
                            deq_b, N, expert_ids, tile_offsets, M, rows, absolute)


# --------------------------------------------------------------------------------------
# a7: MX block-scaled GEMM (e8m0 per 32 K-elements, applied inside the MMA)
# --------------------------------------------------------------------------------------
def mx_gemm(qa, a_scales, qb, b_scales, fmt_a, fmt_b, expert_ids=None, tile_offsets=None,
            rows=None, absolute=False):
    """MX product ``A_ref @ B_ref^T`` with ``X_ref = decode(q) * 2**(scale - 127)``.

    ``qa``: ``[M, K]`` uint8 e4m3, or ``[M, K/2]`` packed e2m1; ``a_scales``
    uint8 ``[M, K/32]``. ``qb``: ``[E, N, K]`` / ``[E, N, K/2]`` (or without the
    expert axis); ``b_scales`` uint8 ``[E, N, K/32]`` (or ``[N, K/32]``).
    """
    qa = np.asarray(qa, np.uint8)
    a_scales = np.asarray(a_scales, np.uint8)
    b_scales = np.asarray(b_scales, np.uint8)
    M = qa.shape[0]
    N = np.asarray(qb).shape[-2]

    def deq_b(e):
        sb = b_scales if b_scales.ndim == 2 else b_scales[e]
        return dequantize_mx(_expert_b(qb, e), sb, fmt_b)

    return _grouped_dequant(lambda r: dequantize_mx(qa[r], a_scales[r], fmt_a),
                            deq_b, N, expert_ids, tile_offsets, M, rows, absolute)


# --------------------------------------------------------------------------------------
# f4: nvfp4 GEMM (e2m1 elements, an e4m3 scale per 16 K-elements)
# --------------------------------------------------------------------------------------
def dequantize_nv(q, scales):
    """``e2m1(q)[r, k] * e4m3(scales[r, k // 16])`` in fp64 (``q`` packed ``[..., K/2]``)."""
    v = decode_elements(q, "e2m1")
    return v * np.repeat(decode_e4m3fn(scales), NV_BLOCK, axis=-1)


def nv_gemm(qa, a_scales, qb, b_scales, expert_ids=None, tile_offsets=None, rows=None,
            absolute=False):
    """nvfp4 product ``A_ref @ B_ref^T`` on the dequantised values (Gluon page,
    ``random_quantized_tensor`` for ``nvfp4`` and the reference of ``make_problem``).

    ``qa``: packed e2m1 ``[M, K/2]``; ``a_scales`` uint8 e4m3 ``[M, K/16]``.
    ``qb``: ``[E, N, K/2]`` (or ``[N, K/2]``); ``b_scales`` uint8 ``[E, N, K/16]``
    (or ``[N, K/16]``). Grouping as in :func:`blockwise_grouped`.
    """
    qa = np.asarray(qa, np.uint8)
    a_scales = np.asarray(a_scales, np.uint8)
    b_scales = np.asarray(b_scales, np.uint8)
    M = qa.shape[0]
    N = np.asarray(qb).shape[-2]

    def deq_b(e):
        sb = b_scales if b_scales.ndim == 2 else b_scales[e]
        return dequantize_nv(_expert_b(qb, e), sb)

    return _grouped_dequant(lambda r: dequantize_nv(qa[r], a_scales[r]), deq_b, N, expert_ids,
                            tile_offsets, M, rows, absolute)


# --------------------------------------------------------------------------------------
# comparison metric
# --------------------------------------------------------------------------------------
def relative_error(c_test, c_ref, denom):
    """``max |c_test - c_ref| / denom`` over elements with ``denom > 0``.

    ``denom`` is ``sum_k |a||b|`` per element. Elements with ``denom == 0``
    must match exactly (returns inf otherwise). Any NaN/Inf in ``c_test``
    returns inf.
    """
    c_test = np.asarray(c_test, np.float64)
    c_ref = np.asarray(c_ref, np.float64)
    denom = np.asarray(denom, np.float64)
    if not np.all(np.isfinite(c_test)):
        return float("inf")
    zero = denom == 0
    if np.any(c_test[zero] != c_ref[zero]):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(np.abs(c_test[~zero] - c_ref[~zero]) / denom[~zero]))
