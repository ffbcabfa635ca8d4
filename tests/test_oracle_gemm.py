"""Pins for the fp64 GEMM oracle (CPU only).

The oracle is checked against things fixed outside it:

* exact rational brute force on tiny grouped and ragged inputs, with operands
  decoded by torch's own float8 conversions (not the oracle's decoders);
* exact power-of-two scale invariance and per-block scale locality;
* closed forms (all-ones operands);
* the rule that the grouped result equals a loop of per-expert dense GEMMs;
* a hand-worked tile map;
* planted mistakes: copies of the promote loop with one plausible bug each
  must fail the brute-force pin that the real oracle passes.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as ofmt
from oracle import gemm as og
from tests.conftest import read_golden
from workloads.generate import blockwise_problem, mx_problem, nv_problem

NAN_CODES = (0x7F, 0xFF)


# --------------------------------------------------------------------------------------
# independent exact helpers
# --------------------------------------------------------------------------------------
def lib_e4m3_int(codes):
    """e4m3 codes -> exact integers v * 2**9, via torch's float8 conversion."""
    f = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float()
    return (f.double() * 512).numpy().astype(np.int64)


def lib_e8m0_exponent(codes):
    f = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e8m0fnu).float()
    return np.log2(f.double().numpy()).round().astype(np.int64)


E2M1_TIMES2 = {int(c): int(round(float(v) * 2)) for c, v in read_golden("mx_e2m1_values.txt")}


def spec_e2m1_int(packed):
    """packed e2m1 -> exact integers v * 2 (golden spec table; even K index = low nibble)."""
    p = np.asarray(packed, np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int64)
    codes[..., 0::2] = p & 0xF
    codes[..., 1::2] = p >> 4
    return np.vectorize(E2M1_TIMES2.get)(codes)


def exact_blockwise(qa, sa, qb, sb, owner):
    """C[m, n] = sum_k qa*sa*qb*sb exactly (Fractions); owner[m] = expert or None."""
    M, K = qa.shape
    N = qb.shape[-2]
    ia = lib_e4m3_int(qa)
    out = {}
    for m in range(M):
        e = owner[m]
        if e is None:
            continue
        ib = lib_e4m3_int(qb[e])
        for n in range(N):
            total = Fraction(0)
            for kb in range(K // 128):
                k = slice(128 * kb, 128 * kb + 128)
                dot = int(np.dot(ia[m, k], ib[n, k]))           # exact integer, * 2**18
                total += Fraction(dot, 1 << 18) * Fraction(float(sa[m, kb])) * Fraction(float(sb[e][n // 128, kb]))
            out[m, n] = total
    return out


def random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[np.isin(c, NAN_CODES)] = 0x38
    return c


def random_scales(rng, shape, lo=-12, hi=12):
    mant = rng.uniform(1.0, 2.0, size=shape)
    return np.ldexp(mant, rng.integers(lo, hi, size=shape)).astype(np.float32)


def ragged_case(seed=0, K=256, N=256):
    """10 rows, 3 experts, ragged tiles: an empty tile, two tiles of one expert, a skipped tile."""
    rng = np.random.default_rng(seed)
    M, E = 10, 3
    qa = random_codes(rng, (M, K))
    sa = random_scales(rng, (M, K // 128))
    qb = random_codes(rng, (E, N, K))
    sb = random_scales(rng, (E, N // 128, K // 128))
    tile_offsets = np.array([0, 3, 3, 7, 9, 10])
    expert_ids = np.array([2, 0, 1, 1, -1])
    owner = [2, 2, 2, 1, 1, 1, 1, 1, 1, None]   # written by hand from the two arrays above
    return qa, sa, qb, sb, expert_ids, tile_offsets, owner


def check_against_exact(fn, K=256, seeds=(0, 1), dot_bound=False):
    """True iff ``fn`` matches exact arithmetic on :func:`ragged_case` inputs.

    One K block: bitwise equal to the correctly rounded exact value. More blocks:
    within (K/128 + 1) fp64 roundings of the scaled block terms' magnitude; with
    ``dot_bound`` (a plain dequantised dot product) within ``K`` roundings of
    ``sum_k |a_k b_k|``, the textbook bound for a length-K dot product."""
    eps = 2.0 ** -52
    for seed in seeds:
        qa, sa, qb, sb, ei, to, owner = ragged_case(seed, K=K)
        C = fn(qa, sa, qb, sb, ei, to)
        exact = exact_blockwise(qa, sa, qb, sb, owner)
        ia_all = lib_e4m3_int(qa)
        for m in range(qa.shape[0]):
            if owner[m] is None:
                if not np.all(np.isnan(C[m])):
                    return False
                continue
            e = owner[m]
            ib_all = lib_e4m3_int(qb[e])
            for n in range(C.shape[1]):
                want = float(exact[m, n])
                if K == 128 and not dot_bound:
                    if C[m, n] != want:
                        return False
                    continue
                ia, ib = ia_all[m], ib_all[n]
                sc = [float(sa[m, b]) * float(sb[e][n // 128, b]) for b in range(K // 128)]
                if dot_bound:
                    mag = sum(float(np.dot(np.abs(ia[128 * b:128 * b + 128]), np.abs(ib[128 * b:128 * b + 128])))
                              * sc[b] for b in range(K // 128)) / 2 ** 18
                    bound = K * eps * mag
                else:
                    mag = sum(abs(int(np.dot(ia[128 * b:128 * b + 128], ib[128 * b:128 * b + 128]))) * sc[b]
                              for b in range(K // 128)) / 2 ** 18
                    bound = (K // 128 + 1) * eps * mag
                if not abs(C[m, n] - want) <= bound:
                    return False
    return True


# --------------------------------------------------------------------------------------
# exact brute force
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("K", [128, 256])
def test_blockwise_matches_exact(K):
    assert check_against_exact(og.blockwise_grouped, K=K)


def test_dequant_definition_matches_exact():
    assert check_against_exact(og.blockwise_grouped_dequant, K=256, dot_bound=True)


# planted mistakes in a copy of the promote loop: each must fail the pin above
def _mutant(bug):
    from oracle.formats import decode_e4m3fn

    def fn(qa, sa, qb, sb, ei, to):
        M, K = qa.shape
        N = qb.shape[1]
        C = np.full((M, N), np.nan)
        owner = og.row_experts(ei, to, M)
        if bug == "ignore_expert_ids":
            owner = np.where(owner >= 0, 0, -1)
        for m in range(M):
            e = owner[m]
            if e < 0:
                continue
            a = decode_e4m3fn(qa[m])
            b = decode_e4m3fn(qb[e])
            acc = np.zeros(N)
            nblocks = K // 128 - (1 if bug == "drop_last_k_block" else 0)
            for kb in range(nblocks):
                blk = slice(128 * kb, 128 * kb + 128)
                if bug == "transposed_b":          # B read as [K, N] (square here)
                    p = b.T[:, blk] @ a[blk]
                elif bug == "k_order_mismatch":    # A and B walk K in opposite orders
                    p = b[:, blk] @ a[blk][::-1]
                else:
                    p = b[:, blk] @ a[blk]
                ncol = 256 if bug == "b_scale_n_block_256" else 128
                bs = sb[e][np.minimum(np.arange(N) // ncol, sb[e].shape[0] - 1), kb]
                akb = 0 if bug == "a_scale_first_block_only" else kb
                s = np.float64(sa[m, akb]) * bs.astype(np.float64)
                if bug == "scale_product_in_fp32":
                    s = (sa[m, akb] * bs).astype(np.float64)
                if bug == "sign_flip_b_scale":
                    s = -s
                acc += p * s
            C[m] = acc
        return C
    return fn


@pytest.mark.parametrize("bug", ["ignore_expert_ids", "drop_last_k_block", "transposed_b",
                                 "k_order_mismatch",
                                 "b_scale_n_block_256", "a_scale_first_block_only",
                                 "sign_flip_b_scale", "scale_product_in_fp32"])
def test_planted_mistakes_are_caught(bug):
    assert check_against_exact(_mutant("none"), K=256, seeds=(0,))
    assert not check_against_exact(_mutant(bug), K=256, seeds=(0,))


# --------------------------------------------------------------------------------------
# invariances and closed forms
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("fn", [og.blockwise_grouped, og.blockwise_grouped_dequant])
@pytest.mark.parametrize("k", [-20, -3, 1, 17])
def test_power_of_two_scale_invariance(fn, k):
    qa, sa, qb, sb, ei, to, owner = ragged_case(3, K=384)
    base = fn(qa, sa, qb, sb, ei, to)
    f = np.float32(2.0 ** k)
    up_a = fn(qa, sa * f, qb, sb, ei, to)
    up_b = fn(qa, sa, qb, sb * f, ei, to)
    live = ~np.isnan(base)
    assert np.array_equal(up_a[live], base[live] * 2.0 ** k)
    assert np.array_equal(up_b[live], base[live] * 2.0 ** k)


def test_b_scale_locality():
    qa, sa, qb, sb, ei, to, owner = ragged_case(4, K=256)
    base = og.blockwise_grouped(qa, sa, qb, sb, ei, to)
    sb2 = sb.copy()
    sb2[1, 1, 0] *= np.float32(3.0)      # expert 1, columns 128..255, K block 0
    changed = og.blockwise_grouped(qa, sa, qb, sb2, ei, to)
    diff = ~((changed == base) | (np.isnan(changed) & np.isnan(base)))
    rows = np.array([o == 1 for o in owner])
    assert not diff[~rows].any()
    assert not diff[:, :128].any()
    assert diff[rows][:, 128:].all()


def test_closed_form_all_ones():
    M, N, K = 4, 256, 512
    qa = np.full((M, K), 0x38, np.uint8)          # e4m3 1.0
    qb = np.full((1, N, K), 0x38, np.uint8)
    alpha = np.array([0.5, 3.0, 0.125, 1.0], np.float32)
    sa = np.repeat(alpha[:, None], K // 128, axis=1)
    sb = np.full((1, N // 128, K // 128), 0.25, np.float32)
    for fn in (og.blockwise_grouped, og.blockwise_grouped_dequant):
        C = fn(qa, sa, qb, sb)
        assert np.array_equal(C, np.repeat((K * alpha.astype(np.float64) * 0.25)[:, None], N, axis=1))


def test_unit_scales_equal_library_matmul():
    """With unit scales the oracle is a plain matmul of the (library-decoded) codes."""
    rng = np.random.default_rng(5)
    qa = random_codes(rng, (16, 256))
    qb = random_codes(rng, (1, 128, 256))
    C = og.blockwise_grouped(qa, np.ones((16, 2), np.float32), qb, np.ones((1, 1, 2), np.float32))
    ref = (lib_e4m3_int(qa).astype(np.float64) @ lib_e4m3_int(qb[0]).T.astype(np.float64)) / 2 ** 18
    assert np.array_equal(C, ref)


def test_grouped_equals_per_expert_dense():
    counts = [5, 0, 130, 17]
    p = blockwise_problem(counts, 256, 384, seed=2)
    qa, sa, qb, sb = (t.numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales))
    eo, to, ei = og.tile_map(counts, p.M // 128)
    C = og.blockwise_grouped(qa, sa, qb, sb, ei, to)
    for e, c in enumerate(counts):
        lo, hi = int(eo[e]), int(eo[e + 1])
        dense = og.blockwise_grouped(qa[lo:lo + c], sa[lo:lo + c], qb[e], sb[e])
        assert np.array_equal(C[lo:lo + c], dense)
        assert np.all(C[lo + c:hi] == 0.0)           # padding rows are exactly zero


def test_rows_subset_matches_full():
    counts = [40, 200]
    p = blockwise_problem(counts, 128, 256, seed=3)
    args = [t.numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales)]
    _, to, ei = og.tile_map(counts, p.M // 128)
    full = og.blockwise_grouped(*args, ei, to)
    rows = [0, 39, 128, 300]
    sub = og.blockwise_grouped(*args, ei, to, rows=rows)
    assert np.array_equal(sub[rows], full[rows])
    others = np.setdiff1d(np.arange(p.M), rows)
    assert np.all(np.isnan(sub[others]))


# --------------------------------------------------------------------------------------
# tile map: hand-worked example
# --------------------------------------------------------------------------------------
def test_tile_map_worked_example_padded():
    eo, to, ei = og.tile_map([3, 0, 130, 128], 6, padded=True)
    assert eo.tolist() == [0, 128, 128, 384, 512]
    assert to.tolist() == [0, 128, 256, 384, 512, 640, 768]
    assert ei.tolist() == [0, 2, 2, 3, -1, -1]


def test_tile_map_worked_example_compact():
    eo, to, ei = og.tile_map([3, 0, 130, 128], 6, padded=False)
    assert eo.tolist() == [0, 3, 3, 133, 261]
    assert to.tolist() == [0, 3, 131, 133, 261, 261, 261]
    assert ei.tolist() == [0, 2, 2, 3, -1, -1]


def test_tile_map_overflow_and_empty():
    eo, to, ei = og.tile_map([300, 5], 2, padded=True)
    assert eo[-1] == 512 and ei.tolist() == [0, 0]          # the layout needs 4 tiles; 2 kept
    eo, to, ei = og.tile_map([0, 0, 0], 3)
    assert eo.tolist() == [0, 0, 0, 0] and ei.tolist() == [-1, -1, -1]


def test_tile_map_covers_every_row_once():
    rng = np.random.default_rng(7)
    for padded in (True, False):
        counts = rng.integers(0, 400, size=9)
        counts[3] = 0
        counts[5] = 256
        T = 40
        eo, to, ei = og.tile_map(counts, T, padded=padded)
        owner = og.row_experts(ei, to, int(to[-1]) if not padded else 128 * T)
        for e, c in enumerate(counts):
            assert np.all(owner[eo[e]:eo[e] + c] == e)
        assert np.sum(owner >= 0) == (np.sum(-(-counts // 128) * 128) if padded else counts.sum())


# --------------------------------------------------------------------------------------
# MX
# --------------------------------------------------------------------------------------
def exact_mx(qa, sa, qb, sb, fa, fb):
    def ints(q, f):
        return (lib_e4m3_int(q), 512) if f == "e4m3" else (spec_e2m1_int(q), 2)

    ia, da = ints(qa, fa)
    ib, db = ints(qb, fb)
    ea, eb = lib_e8m0_exponent(sa), lib_e8m0_exponent(sb)
    M, K = ia.shape
    N = ib.shape[0]
    out = np.empty((M, N), object)
    for m in range(M):
        for n in range(N):
            t = Fraction(0)
            for j in range(K // 32):
                k = slice(32 * j, 32 * j + 32)
                t += Fraction(int(np.dot(ia[m, k], ib[n, k])), da * db) * Fraction(2) ** int(ea[m, j] + eb[n, j])
            out[m, n] = t
    return out


@pytest.mark.parametrize("fa,fb", [("e2m1", "e2m1"), ("e4m3", "e2m1"), ("e4m3", "e4m3")])
def test_mx_matches_exact(fa, fb):
    """Inputs in the style of the Gluon page's random_quantized_tensor: random element
    codes with random e8m0 scales near 1, so every sum is exactly representable."""
    rng = np.random.default_rng(11)
    M, N, K = 6, 8, 128

    def elems(rows, f):
        if f == "e4m3":
            c = random_codes(rng, (rows, K))
            # keep magnitudes small so 128-term sums stay exact in fp64
            return np.where(np.abs(lib_e4m3_int(c)) > 4096, 0x38, c).astype(np.uint8)
        return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)

    qa, qb = elems(M, fa), elems(N, fb)
    sa = rng.integers(120, 131, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 131, size=(N, K // 32)).astype(np.uint8)
    C = og.mx_gemm(qa, sa, qb, sb, fa, fb)
    want = exact_mx(qa, sa, qb, sb, fa, fb)
    for m in range(M):
        for n in range(N):
            assert C[m, n] == float(want[m, n])


def test_mx_scale_code_shift():
    p = mx_problem(8, 128, 256, "e4m3", "e2m1", seed=4)
    qa, sa, qb, sb = (t.numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales))
    base = og.mx_gemm(qa, sa, qb[0], sb[0], "e4m3", "e2m1")
    shifted = og.mx_gemm(qa, sa + 3, qb[0], sb[0], "e4m3", "e2m1")
    assert np.array_equal(shifted, base * 8.0)


def test_mx_unit_scales_equal_blockwise_unit_scales():
    rng = np.random.default_rng(6)
    qa = random_codes(rng, (8, 256))
    qb = random_codes(rng, (128, 256))
    mx = og.mx_gemm(qa, np.full((8, 8), 127, np.uint8), qb, np.full((128, 8), 127, np.uint8),
                    "e4m3", "e4m3")
    bw = og.blockwise_grouped(qa, np.ones((8, 2), np.float32), qb, np.ones((1, 2), np.float32))
    assert np.array_equal(mx, bw)


# --------------------------------------------------------------------------------------
# nvfp4 (e2m1 elements, e4m3 scale per 16 K)
# --------------------------------------------------------------------------------------
def exact_nv(qa, sa, qb, sb):
    """Exact Fractions: element ints from the golden e2m1 table, scales via torch's e4m3."""
    ia, ib = spec_e2m1_int(qa), spec_e2m1_int(qb)             # value * 2
    ja, jb = lib_e4m3_int(sa), lib_e4m3_int(sb)               # scale * 512
    M, K = ia.shape
    N = ib.shape[0]
    out = np.empty((M, N), object)
    for m in range(M):
        for n in range(N):
            t = 0
            for j in range(K // 16):
                k = slice(16 * j, 16 * j + 16)
                t += int(np.dot(ia[m, k], ib[n, k])) * int(ja[m, j]) * int(jb[n, j])
            out[m, n] = Fraction(t, 2 * 2 * 512 * 512)
    return out


def random_nv(rng, M, N, K, signed_scales=True):
    qa = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qb = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sa, sb = random_codes(rng, (M, K // 16)), random_codes(rng, (N, K // 16))
    if not signed_scales:
        sa, sb = sa & 0x7F, sb & 0x7F
    return qa, sa, qb, sb


def test_nv_matches_exact():
    """Every e2m1 byte and every finite e4m3 scale code (subnormal, negative and 448 included):
    with K = 128 each sum is exact in fp64, so the oracle must equal the rational result."""
    rng = np.random.default_rng(21)
    qa, sa, qb, sb = random_nv(rng, 6, 8, 128)
    C = og.nv_gemm(qa, sa, qb, sb)
    want = exact_nv(qa, sa, qb, sb)
    for m in range(6):
        for n in range(8):
            assert C[m, n] == float(want[m, n])


def _nv_mutant(bug):
    def deq(q, s, side="b"):
        codes = ofmt.unpack_e2m1(q)
        if bug == "nibble_order" and side == "a":   # on both operands it would cancel
            codes = codes.reshape(codes.shape[:-1] + (-1, 2))[..., ::-1].reshape(codes.shape)
        v = ofmt.decode_e2m1(codes)
        if bug == "scale_block_32":
            sc = np.repeat(ofmt.decode_e4m3fn(s), 32, axis=-1)[..., :v.shape[-1]]
        elif bug == "e8m0_scales":
            sc = np.repeat(ofmt.decode_e8m0(s), 16, axis=-1)
        else:
            sc = np.repeat(ofmt.decode_e4m3fn(s), 16, axis=-1)
        return v * sc

    def fn(qa, sa, qb, sb):
        a, b = deq(qa, sa, "a"), deq(qb, sb)
        if bug == "scales_swapped":
            a, b = deq(qa, sb[: qa.shape[0]]), deq(qb, sa[: qb.shape[0]])
        return a @ b.T

    return fn


@pytest.mark.parametrize("bug", ["nibble_order", "scale_block_32", "e8m0_scales", "scales_swapped"])
def test_nv_planted_mistakes_are_caught(bug):
    rng = np.random.default_rng(22)
    qa, sa, qb, sb = random_nv(rng, 6, 6, 128, signed_scales=False)
    want = exact_nv(qa, sa, qb, sb)
    got = _nv_mutant(bug)(qa, sa, qb, sb)
    assert any(got[m, n] != float(want[m, n]) for m in range(6) for n in range(6))


def test_nv_power_of_two_scales_equal_mx():
    """Scales that are powers of two and equal over each 32 K-elements: the nvfp4 product must
    equal the MX product with the matching e8m0 codes (a different scale decoder)."""
    rng = np.random.default_rng(23)
    M, N, K = 8, 128, 256
    qa = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qb = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ea = rng.integers(-9, 9, size=(M, K // 32))
    eb = rng.integers(-9, 9, size=(N, K // 32))
    # e4m3 code of 2**e: normal (exponent field e + 7) for e >= -6, else subnormal 2**(e+9) * 2**-9
    def e4m3_pow2(e):
        return np.where(e >= -6, (e + 7) << 3, 1 << (e + 9)).astype(np.uint8)
    nv = og.nv_gemm(qa, np.repeat(e4m3_pow2(ea), 2, axis=1), qb, np.repeat(e4m3_pow2(eb), 2, axis=1))
    mx = og.mx_gemm(qa, (ea + 127).astype(np.uint8), qb, (eb + 127).astype(np.uint8), "e2m1", "e2m1")
    assert np.array_equal(nv, mx)


def test_nv_scale_code_shift():
    """Adding 8 to a normal e4m3 code raises its exponent by one: C doubles exactly."""
    p = nv_problem(8, 128, 256, seed=5)
    qa, sa, qb, sb = (t.numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales))
    assert np.all((sa >> 3) & 0xF >= 1) and np.all((sa >> 3) & 0xF <= 13)
    base = og.nv_gemm(qa, sa, qb[0], sb[0])
    assert np.array_equal(og.nv_gemm(qa, sa + 8, qb[0], sb[0]), base * 2.0)


def test_nv_grouped_equals_per_expert_dense():
    p = nv_problem(0, 128, 256, seed=6, counts=[5, 0, 131, 40])
    qa, sa, qb, sb = (t.numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales))
    _, to, ei = og.tile_map(p.counts, p.M // 128)
    C = og.nv_gemm(qa, sa, qb, sb, ei, to)
    owner = og.row_experts(ei, to, p.M)
    for e in range(4):
        r = np.nonzero(owner == e)[0]
        if len(r):
            assert np.array_equal(C[r], og.nv_gemm(qa[r], sa[r], qb[e], sb[e]))
    assert np.all(np.isnan(C[owner < 0]))


def test_nv_quantiser_round_trip_bound():
    """The input encoder keeps every element within half an e2m1 step (times the scale)."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(16, 256, generator=g)
    from workloads.generate import quantize_nvfp4
    q, s = quantize_nvfp4(x)
    deq = og.dequantize_nv(q.numpy(), s.numpy())
    sc = np.repeat(ofmt.decode_e4m3fn(s.numpy()), 16, axis=-1)
    xs = np.abs(x.numpy() / sc)
    step = np.where(xs < 2, 0.5, np.where(xs < 4, 1.0, 2.0))
    assert np.all(np.abs(deq - x.numpy()) <= (step / 2 + 1e-6) * sc + np.maximum(xs - 6, 0) * sc)


# --------------------------------------------------------------------------------------
# metric
# --------------------------------------------------------------------------------------
def test_relative_error_rules():
    ref = np.array([[1.0, 0.0], [2.0, 5.0]])
    den = np.array([[2.0, 0.0], [4.0, 10.0]])
    assert og.relative_error(ref, ref, den) == 0.0
    assert og.relative_error(ref + [[0.02, 0], [0, 0]], ref, den) == pytest.approx(0.01)
    assert og.relative_error(ref + [[0, 1e-30], [0, 0]], ref, den) == float("inf")
    bad = ref.copy()
    bad[1, 1] = np.nan
    assert og.relative_error(bad, ref, den) == float("inf")
