"""Seeded synthetic workloads: routing, quantised operands and scales.

Recipes (all seeded; ``seed`` defaults to 0):

* Values are float32 ~ N(0, 1) drawn with a ``torch.Generator`` on the target
  device, A first, then B. The same seed on another device gives other (but
  again fixed) bytes; every consumer reads the bytes produced here.
* Blockwise e4m3: A gets one fp32 scale ``amax / 448`` per row per 128-wide K
  block, B one per 128x128 block; an all-zero block gets scale 1.
  ``q = e4m3(clamp(x / s, -448, 448))`` with round-to-nearest-even (torch's
  cast).
* MX: one e8m0 code per 32 K-elements, ``floor(log2 amax) - emax + 127``
  (``emax`` = 8 for e4m3, 2 for e2m1; ``floor(log2)`` taken from ``frexp``),
  clamped to [0, 254]; elements ``x * 2**-(code - 127)`` rounded to nearest-even
  and saturated to +-448 (e4m3) or +-6 (e2m1). e2m1 is packed two per byte
  along K, even K index in the low nibble.
* nvfp4: one e4m3 scale per 16 K-elements, ``e4m3(amax / 6)`` rounded to
  nearest-even (an all-zero block gets scale 1, a scale that rounds to zero the
  smallest subnormal); elements ``x / scale`` (fp32) rounded to nearest-even
  e2m1 and saturated to +-6, packed as for MX.
* Routing: ``p ~ Dirichlet(alpha)`` over the experts (``n_empty`` of them
  forced to zero and ``p`` renormalised), ``tokens * top_k`` rows split by
  largest remainder, each count capped at ``tokens`` (a token picks an expert
  at most once) with the surplus refilled over the uncapped experts.
* Grouped layout: experts in ascending order, each group starting at a
  multiple of 128 rows; padding rows are zero with scale 1.
* Token picks (for the quantise-and-permute step): the routing counts dealt
  column-wise over ``tokens x top_k`` so each token's experts are distinct,
  then token and slot order shuffled; activations bf16 from N(0, 1).

Nothing here computes the GEMM or its tile map.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0
EMAX = {"e4m3": 8, "e2m1": 2}


# --------------------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------------------
def _largest_remainder(weights, total):
    raw = weights / weights.sum() * total
    base = np.floor(raw).astype(np.int64)
    short = int(total - base.sum())
    order = np.argsort(-(raw - base), kind="stable")
    base[order[:short]] += 1
    return base


def routing_counts(tokens, top_k, experts, alpha, n_empty=0, seed=0):
    """Per-expert row counts summing to ``tokens * top_k``, each at most ``tokens``."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(experts, float(alpha)))
    if n_empty:
        p[rng.choice(experts, n_empty, replace=False)] = 0.0
    total = tokens * top_k
    counts = _largest_remainder(p, total)
    fixed = np.zeros(experts, bool)
    while np.any(counts > tokens):
        over = counts > tokens
        surplus = int((counts[over] - tokens).sum())
        counts[over] = tokens
        fixed |= over
        free = (~fixed) & (p > 0)
        if not free.any():
            raise ValueError("routing cannot satisfy the per-expert cap")
        counts[free] += _largest_remainder(p[free], surplus)
    assert counts.sum() == total
    return counts


def routing_topk(counts, tokens, top_k, seed=0):
    """Top-k picks ``int32 [tokens, top_k]`` (distinct experts per token) whose per-expert
    totals are ``counts`` (each at most ``tokens``, summing to ``tokens * top_k``).

    The expert ids sorted by expert are dealt column-wise (pick i goes to token i % tokens,
    slot i // tokens), so one expert's picks land on distinct tokens; token order and the
    order of each token's slots are then shuffled (seeded)."""
    counts = np.asarray(counts, dtype=np.int64)
    if counts.sum() != tokens * top_k or np.any(counts > tokens) or np.any(counts < 0):
        raise ValueError("counts must sum to tokens * top_k with each count <= tokens")
    rng = np.random.default_rng(seed + 1)
    flat = np.repeat(np.arange(len(counts)), counts)
    ids = flat.reshape(top_k, tokens).T.copy()
    ids = ids[rng.permutation(tokens)]
    ids = np.take_along_axis(ids, np.argsort(rng.random(ids.shape), axis=1), axis=1)
    return ids.astype(np.int32)


def activations(tokens, K, device="cpu", seed=0, dtype=torch.bfloat16):
    """Token activations ~ N(0, 1), ``[tokens, K]`` in ``dtype`` (bf16 by default)."""
    gen = torch.Generator(device=device).manual_seed(seed + 2)
    return torch.randn(tokens, K, generator=gen, device=device).to(dtype)


def padded_starts(counts, tile=128):
    """First row of each expert's group in the padded layout, plus the total."""
    sizes = [-(-int(c) // tile) * tile for c in counts]
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


# --------------------------------------------------------------------------------------
# quantisers (input encoding only)
# --------------------------------------------------------------------------------------
def _to_e4m3_bytes(y):
    return y.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_e4m3_rowblocks(x):
    """fp32 ``[R, K]`` -> (uint8 e4m3 ``[R, K]``, fp32 scales ``[R, K/128]``)."""
    R, K = x.shape
    xb = x.reshape(R, K // 128, 128)
    amax = xb.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = _to_e4m3_bytes(xb / s[..., None]).reshape(R, K)
    return q, s.contiguous()


def quantize_e4m3_tiles(x):
    """fp32 ``[..., N, K]`` -> (uint8 e4m3 ``[..., N, K]``, fp32 ``[..., N/128, K/128]``)."""
    *lead, N, K = x.shape
    xb = x.reshape(*lead, N // 128, 128, K // 128, 128)
    amax = xb.abs().amax(dim=(-3, -1))
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = _to_e4m3_bytes(xb / s[..., :, None, :, None]).reshape(*lead, N, K)
    return q, s.contiguous()


def _e2m1_codes(y):
    """fp32 -> e2m1 codes (0..15), nearest-even, saturating at 6."""
    a = y.abs()
    mag = ((a > 0.25).to(torch.int32) + (a >= 0.75).to(torch.int32) + (a > 1.25).to(torch.int32)
           + (a >= 1.75).to(torch.int32) + (a > 2.5).to(torch.int32) + (a >= 3.5).to(torch.int32)
           + (a > 5.0).to(torch.int32))
    return mag | ((y < 0).to(torch.int32) << 3)


def pack_e2m1(codes):
    """int codes ``[..., K]`` -> uint8 ``[..., K/2]`` (even K index in the low nibble)."""
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).to(torch.uint8)


def quantize_mx(x, fmt):
    """fp32 ``[..., R, K]`` -> (elements, uint8 e8m0 ``[..., R, K/32]``).

    Elements are uint8 e4m3 ``[..., R, K]`` or packed e2m1 ``[..., R, K/2]``.
    """
    *lead, K = x.shape
    xb = x.reshape(*lead, K // 32, 32)
    amax = xb.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                     # amax = m * 2**ex, m in [0.5, 1)
    code = (ex - 1 - EMAX[fmt] + 127).clamp(0, 254)
    code = torch.where(amax > 0, code, torch.full_like(code, 127))
    y = torch.ldexp(xb, -(code - 127).to(torch.float32)[..., None])
    if fmt == "e4m3":
        q = _to_e4m3_bytes(y).reshape(*lead, K)
    elif fmt == "e2m1":
        q = pack_e2m1(_e2m1_codes(y.clamp(-E2M1_MAX, E2M1_MAX)).reshape(*lead, K))
    else:
        raise ValueError(fmt)
    return q, code.to(torch.uint8).contiguous()


def quantize_nvfp4(x):
    """fp32 ``[..., R, K]`` -> (packed e2m1 ``[..., R, K/2]``, uint8 e4m3 ``[..., R, K/16]``)."""
    *lead, K = x.shape
    xb = x.reshape(*lead, K // 16, 16)
    amax = xb.abs().amax(dim=-1)
    code = _to_e4m3_bytes(amax / E2M1_MAX)
    code = torch.where(amax > 0, code, torch.full_like(code, 0x38))     # 1.0
    code = torch.where(code == 0, torch.ones_like(code), code)          # smallest subnormal
    s = code.view(torch.float8_e4m3fn).float()
    y = (xb / s[..., None]).clamp(-E2M1_MAX, E2M1_MAX)
    q = pack_e2m1(_e2m1_codes(y).reshape(*lead, K))
    return q, code.contiguous()


# --------------------------------------------------------------------------------------
# problems
# --------------------------------------------------------------------------------------
@dataclass
class Problem:
    """One GEMM instance: quantised operands plus the routing they came from."""

    name: str
    scale_kind: str            # "blockwise" (fp32 1x128 / 128x128), "mx" (e8m0 per 32) or
                               # "nv" (e4m3 per 16, e2m1 elements)
    fmt_a: str                 # "e4m3" | "e2m1"
    fmt_b: str
    out_dtypes: tuple          # subset of ("f32", "bf16", "f16")
    M: int                     # rows of A (padded layout)
    N: int
    K: int
    E: int
    counts: Optional[np.ndarray]  # per-expert real rows, None for one dense group
    qa: torch.Tensor
    a_scales: torch.Tensor
    qb: torch.Tensor           # [E, N, K] (or [E, N, K/2] packed e2m1)
    b_scales: torch.Tensor
    meta: dict = field(default_factory=dict)

    @property
    def real_rows(self):
        return int(self.M if self.counts is None else int(np.sum(self.counts)))

    @property
    def useful_flops(self):
        return 2.0 * self.real_rows * self.N * self.K


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _blockwise_problem(name, counts, N, K, E, out_dtypes, device, seed, outlier_every=0,
                       a_rows=None):
    gen = torch.Generator(device=device).manual_seed(seed)
    if counts is None:
        M = int(a_rows)
        x = _randn((M, K), gen, device)
        if outlier_every:
            x[::outlier_every] *= 100.0
        qa, sa = quantize_e4m3_rowblocks(x)
        del x
    else:
        starts = padded_starts(counts)
        M = int(starts[-1])
        qa = torch.zeros((M, K), dtype=torch.uint8, device=device)
        sa = torch.ones((M, K // 128), dtype=torch.float32, device=device)
        for e, c in enumerate(counts):
            c = int(c)
            if c == 0:
                continue
            x = _randn((c, K), gen, device)
            q, s = quantize_e4m3_rowblocks(x)
            qa[starts[e]:starts[e] + c] = q
            sa[starts[e]:starts[e] + c] = s
            del x, q, s
    qbs, sbs = [], []
    for _ in range(E):
        y = _randn((N, K), gen, device)
        if outlier_every:
            y[::outlier_every] *= 100.0
        q, s = quantize_e4m3_tiles(y)
        qbs.append(q)
        sbs.append(s)
        del y
    qb = torch.stack(qbs)
    sb = torch.stack(sbs)
    return Problem(name, "blockwise", "e4m3", "e4m3", out_dtypes, M, N, K, E,
                   None if counts is None else np.asarray(counts, np.int64), qa, sa, qb, sb)


def _mx_problem(name, M, N, K, fmt_a, fmt_b, device, seed):
    gen = torch.Generator(device=device).manual_seed(seed)
    qa, sa = quantize_mx(_randn((M, K), gen, device), fmt_a)
    qb, sb = quantize_mx(_randn((N, K), gen, device), fmt_b)
    return Problem(name, "mx", fmt_a, fmt_b, ("f16",), M, N, K, 1, None, qa, sa,
                   qb[None].contiguous(), sb[None].contiguous())


def _nv_problem(name, M, N, K, device, seed, counts=None, E=1):
    """nvfp4 operands: one dense group of M rows, or grouped (padded layout) from ``counts``."""
    gen = torch.Generator(device=device).manual_seed(seed)
    if counts is None:
        qa, sa = quantize_nvfp4(_randn((M, K), gen, device))
    else:
        starts = padded_starts(counts)
        M = int(starts[-1])
        qa = torch.zeros((M, K // 2), dtype=torch.uint8, device=device)
        sa = torch.full((M, K // 16), 0x38, dtype=torch.uint8, device=device)
        for e, c in enumerate(counts):
            c = int(c)
            if c:
                qa[starts[e]:starts[e] + c], sa[starts[e]:starts[e] + c] = quantize_nvfp4(
                    _randn((c, K), gen, device))
        E = len(counts)
    qb, sb = quantize_nvfp4(_randn((E, N, K), gen, device))
    return Problem(name, "nv", "e2m1", "e2m1", ("f16",), M, N, K, E,
                   None if counts is None else np.asarray(counts, np.int64), qa, sa,
                   qb.contiguous(), sb.contiguous())


MOE8 = dict(tokens=4096, top_k=2, experts=8, alpha=0.5, n_empty=0)
MOE32 = dict(tokens=16384, top_k=8, experts=32, alpha=1.0, n_empty=2)

WORKLOADS = {
    # one expert, 128 x 256 x 512, fp32 and bf16 output
    "single_128x256x512": lambda dev, seed: _blockwise_problem(
        "single_128x256x512", None, 256, 512, 1, ("f32", "bf16"), dev, seed, a_rows=128),
    # one dense group 4096^3, every 64th row of A and of B scaled x100, bf16 output
    "dense_4096": lambda dev, seed: _blockwise_problem(
        "dense_4096", None, 4096, 4096, 1, ("bf16",), dev, seed, outlier_every=64, a_rows=4096),
    # one dense group with few 256 x 256 tiles and a long K (8 tiles, K = 16384), bf16 output
    "dense_256x2048x16384": lambda dev, seed: _blockwise_problem(
        "dense_256x2048x16384", None, 2048, 16384, 1, ("bf16",), dev, seed, a_rows=256),
    # 8 experts, 4096 tokens top-2, Dirichlet(0.5), N=2048, K=4096, bf16
    "moe8_n2048_k4096": lambda dev, seed: _blockwise_problem(
        "moe8_n2048_k4096", routing_counts(seed=seed, **MOE8), 2048, 4096, 8, ("bf16",), dev, seed),
    # 32 local experts, 16384 tokens top-8, Dirichlet(1.0), two experts empty, bf16
    "moe32_gate_up_n4096_k7168": lambda dev, seed: _blockwise_problem(
        "moe32_gate_up_n4096_k7168", routing_counts(seed=seed, **MOE32), 4096, 7168, 32, ("bf16",),
        dev, seed),
    "moe32_down_n7168_k2048": lambda dev, seed: _blockwise_problem(
        "moe32_down_n7168_k2048", routing_counts(seed=seed, **MOE32), 7168, 2048, 32, ("bf16",),
        dev, seed + 1),
    # MX 8192^3, three element-format pairs, fp16 output
    "mx8192_e4m3_e4m3": lambda dev, seed: _mx_problem("mx8192_e4m3_e4m3", 8192, 8192, 8192,
                                                      "e4m3", "e4m3", dev, seed),
    "mx8192_e4m3_e2m1": lambda dev, seed: _mx_problem("mx8192_e4m3_e2m1", 8192, 8192, 8192,
                                                      "e4m3", "e2m1", dev, seed),
    "mx8192_e2m1_e2m1": lambda dev, seed: _mx_problem("mx8192_e2m1_e2m1", 8192, 8192, 8192,
                                                      "e2m1", "e2m1", dev, seed),
    # nvfp4 (e2m1, e4m3 scale per 16 K) 8192^3, fp16 output
    "nvfp4_8192": lambda dev, seed: _nv_problem("nvfp4_8192", 8192, 8192, 8192, dev, seed),
}


def make_problem(name, device="cpu", seed=0):
    """Build a named workload on ``device``."""
    return WORKLOADS[name](device, seed)


def blockwise_problem(counts, N, K, device="cpu", seed=0, a_rows=None, E=None, outlier_every=0,
                      out_dtypes=("f32", "bf16")):
    """Ad-hoc blockwise problem (tests): grouped if ``counts`` is given, else dense."""
    E = len(counts) if counts is not None else (E or 1)
    return _blockwise_problem("adhoc", counts, N, K, E, out_dtypes, device, seed,
                              outlier_every=outlier_every, a_rows=a_rows)


def nv_problem(M, N, K, device="cpu", seed=0, counts=None):
    """Ad-hoc nvfp4 problem (tests): dense (M rows) or grouped from ``counts``."""
    return _nv_problem("adhoc_nv", M, N, K, device, seed, counts=counts)


def mx_problem(M, N, K, fmt_a, fmt_b, device="cpu", seed=0):
    """Ad-hoc single-group MX problem (tests)."""
    return _mx_problem("adhoc_mx", M, N, K, fmt_a, fmt_b, device, seed)
