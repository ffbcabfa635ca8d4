"""Shared GPU-vs-oracle parity machinery for the ``gpu`` tests.

The HIP path runs through the C ABI (via the thin binding); the oracle runs on the CPU on
the same input bytes, with its own tile map. Tolerances (error measured against
``D = sum_k |a||b|`` per element): 1e-3 for fp32 and fp16 output, 8e-3 for bf16 output.
"""

import sys

import numpy as np
import torch

import mx_grouped_gemm_amd as bsg
from oracle import gemm as og

TOL = {"f32": 1e-3, "bf16": 8e-3, "f16": 1e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def poisoned(M, N, out, device="cuda"):
    return torch.full((M, N), float("nan"), dtype=bsg.OUT_DTYPE[out], device=device)


def gpu_tile_map(counts, num_tiles, padded=True):
    c = torch.as_tensor(np.asarray(counts, np.int32), device="cuda")
    eo, to, ei = bsg.bsgemm_build_tiles(c, num_tiles, padded=padded)
    return eo, to, ei


def run_problem(prob, out, tile_map=None, num_tiles=None):
    """Run the HIP path on a workloads.Problem. ``tile_map`` = (expert_ids, tile_offsets) device
    tensors, or None to build it on the GPU from ``prob.counts`` (dense if counts is None)."""
    if tile_map is None and prob.counts is not None:
        T = num_tiles if num_tiles is not None else prob.M // 128
        _, to, ei = gpu_tile_map(prob.counts, T)
        tile_map = (ei, to)
    ei, to = tile_map if tile_map is not None else (None, None)
    C = poisoned(prob.M, prob.N, out)
    fmt = bsg.make_fmt(prob.fmt_a, prob.fmt_b, prob.scale_kind, out)
    bsg.bsgemm_grouped(prob.qa, prob.a_scales, prob.qb, prob.b_scales, ei, to, C, prob.M, prob.N,
                       prob.K, fmt, num_tiles=None if ei is None else ei.numel(),
                       num_experts=prob.E)
    return C, ei, to


def oracle_reference(prob, expert_ids, tile_offsets, rows=None):
    """(C_ref, D) from the oracle, on the CPU, for the given rows (all if None)."""
    qa, sa, qb, sb = (t.cpu().numpy() for t in (prob.qa, prob.a_scales, prob.qb, prob.b_scales))
    if prob.scale_kind == "blockwise":
        ref = og.blockwise_grouped(qa, sa, qb, sb, expert_ids, tile_offsets, rows=rows)
        den = og.blockwise_grouped_dequant(qa, sa, qb, sb, expert_ids, tile_offsets, rows=rows,
                                           absolute=True)
    elif prob.scale_kind == "nv":
        ref = og.nv_gemm(qa, sa, qb, sb, expert_ids, tile_offsets, rows=rows)
        den = og.nv_gemm(qa, sa, qb, sb, expert_ids, tile_offsets, rows=rows, absolute=True)
    else:
        ref = og.mx_gemm(qa, sa, qb, sb, prob.fmt_a, prob.fmt_b, expert_ids, tile_offsets, rows=rows)
        den = og.mx_gemm(qa, sa, qb, sb, prob.fmt_a, prob.fmt_b, expert_ids, tile_offsets, rows=rows,
                         absolute=True)
    return ref, den


def check(prob, out, C_gpu, rows=None, tile_map_ref=None, label=""):
    """Compare the GPU output with the oracle; rows the oracle leaves uncovered must still hold
    the NaN poison. Returns the max relative error."""
    if tile_map_ref is None:
        if prob.counts is None:
            ei_ref, to_ref = None, None
        else:
            _, to_ref, ei_ref = og.tile_map(prob.counts, prob.M // 128)
    else:
        ei_ref, to_ref = tile_map_ref
    ref, den = oracle_reference(prob, ei_ref, to_ref, rows)
    C = C_gpu.float().cpu().numpy().astype(np.float64)
    sel = np.arange(prob.M) if rows is None else np.unique(np.asarray(rows))
    covered = og.row_experts(ei_ref, to_ref, prob.M)[sel] >= 0
    live = sel[covered]
    dead = sel[~covered]
    assert np.all(np.isnan(C[dead])), f"{label}: rows outside every tile were written"
    err = og.relative_error(C[live], ref[live], den[live]) if len(live) else 0.0
    say(f"[parity] {label} out={out} rows={len(live)} max_rel_err={err:.3e} tol={TOL[out]:.0e}")
    assert err <= TOL[out], f"{label}: max relative error {err} > {TOL[out]}"
    return err


def sample_rows(prob, per_tile=12, seed=0):
    """Rows of every 128-row tile to compare: the first and the last, one row in each of the
    tile's eight 16-row fragment bands, and ``per_tile - 10`` random rows. Band b gives row
    16 b + 2 b or 16 b + 2 b + 1 (at random), so that the eight rows cover all eight classes of
    (r >> 1) & 7 (the LDS slot swizzle of the staged A scales) and of (r >> 3) & 7 (the row bits
    above a fragment's 8-row half)."""
    rng = np.random.default_rng(seed)
    rows = []
    for t in range(0, prob.M, 128):
        hi = min(t + 128, prob.M)
        cand = [t, hi - 1]
        cand += [t + 16 * b + 2 * b + int(rng.integers(0, 2)) for b in range(8)]
        cand += [int(r) for r in rng.integers(t, hi, size=max(per_tile - 10, 0))]
        rows += [r for r in cand if r < hi]
    return np.unique(rows)
