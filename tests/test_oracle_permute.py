"""Pins of the quantise-and-permute oracle against facts that do not come from the oracle itself:
the e4m3fn grid (every code, every midpoint), torch's own float8_e4m3fn conversion, the
power-of-two behaviour of a block scale, the rounding error bound, and a sort-based
construction of the row permutation."""

import numpy as np
import pytest
import torch

from oracle import formats, permute

NON_NAN = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_encode_round_trips_every_code():
    codes = np.array(NON_NAN, dtype=np.uint8)
    vals = formats.decode_e4m3fn(codes)
    assert np.array_equal(permute.encode_e4m3fn(vals), codes)


def test_encode_ties_go_to_even_codes():
    pos = np.array([c for c in NON_NAN if c < 0x7F], dtype=np.int64)
    lo, hi = pos[:-1], pos[1:]
    mid = (formats.decode_e4m3fn(lo) + formats.decode_e4m3fn(hi)) / 2      # exact in fp64
    got = permute.encode_e4m3fn(mid).astype(np.int64)
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, want)
    # one fp64 step either side of the midpoint goes to the nearer code
    assert np.array_equal(permute.encode_e4m3fn(np.nextafter(mid, 0)).astype(np.int64), lo)
    assert np.array_equal(permute.encode_e4m3fn(np.nextafter(mid, 1e9)).astype(np.int64), hi)
    # and negative values mirror
    assert np.array_equal(permute.encode_e4m3fn(-mid).astype(np.int64), want | 0x80)


def test_encode_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(5)
    mags = np.concatenate([rng.uniform(0, 448, 40000), rng.uniform(0, 2.0 ** -6, 20000),
                           np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448), 40000))])
    v = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    v = np.clip(v, -448, 448)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(permute.encode_e4m3fn(v), lib)


def test_encode_signed_zero():
    assert permute.encode_e4m3fn(np.array([0.0, -0.0, -2.0 ** -11]))[1:].tolist() == [0x80, 0x80]
    assert permute.encode_e4m3fn(np.array([0.0]))[0] == 0


def _rows(seed, R=6, K=384):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)).astype(np.float32)
    x[1, 128:256] = 0.0                                   # an all-zero block
    x[2] *= 1e-30                                         # tiny values: scale in fp32 normals
    x[3, 5] = 1e4                                         # an outlier dominating its block
    return x


def test_quantize_rows_block_max_maps_to_448():
    x = _rows(1)
    q, s = permute.quantize_rows(x)
    R, K = x.shape
    for r in range(R):
        for b in range(K // 128):
            blk = x[r, 128 * b:128 * b + 128]
            if not np.any(blk):
                assert s[r, b] == 1.0 and not np.any(q[r, 128 * b:128 * b + 128])
                continue
            i = int(np.argmax(np.abs(blk)))
            assert q[r, 128 * b + i] & 0x7F == 0x7E      # +-448


def test_quantize_rows_power_of_two_invariance():
    x = _rows(2)
    q0, s0 = permute.quantize_rows(x)
    for k in (-7, -1, 3, 11):
        q, s = permute.quantize_rows(x * np.float32(2.0 ** k))
        assert np.array_equal(q, q0)
        nz = s0 != 1.0                                    # all-zero blocks keep scale 1
        assert np.array_equal(s[nz], s0[nz] * np.float32(2.0 ** k)) and np.all(s[~nz] == 1.0)


def test_quantize_rows_error_bound():
    """Round to nearest on the e4m3 grid: error <= half a step, i.e. <= 2**-4 of the value for
    normals and <= 2**-10 (times the scale) in the subnormal range."""
    x = _rows(3)
    q, s = permute.quantize_rows(x)
    deq = formats.decode_e4m3fn(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(x.astype(np.float64)), 2.0 ** -10 * sc) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)


def test_route_counts_and_dest_against_a_stable_sort():
    rng = np.random.default_rng(7)
    T, k, E = 200, 3, 9
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[5, 1] = -1                                        # dropped pick
    ids[9, 0] = E                                         # out-of-range id
    counts = permute.route_counts(ids, E)
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    assert np.array_equal(counts, np.bincount(flat[ok], minlength=E))
    pad = -(-counts // 128) * 128
    offs = np.concatenate([[0], np.cumsum(pad)]).astype(np.int64)
    dest = permute.permute_dest(ids, offs, int(offs[-1])).reshape(-1)
    # independent construction: stable sort of the valid picks by expert id
    picks = np.nonzero(ok)[0]
    order = picks[np.argsort(flat[picks], kind="stable")]
    want = np.full(flat.size, -1)
    for e in range(E):
        mine = order[flat[order] == e]
        want[mine] = offs[e] + np.arange(len(mine))
    assert np.array_equal(dest, want)


def test_quantize_permute_rows_and_padding():
    rng = np.random.default_rng(8)
    T, k, E, K = 50, 2, 4, 256
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, K)).astype(np.float32)
    counts = permute.route_counts(ids, E)
    offs = np.concatenate([[0], np.cumsum(-(-counts // 128) * 128)])
    M = int(offs[-1])
    dest, qa, sa, written = permute.quantize_permute(x, ids, offs, M)
    q, s = permute.quantize_rows(x)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(qa[dest[t, j]], q[t]) and np.array_equal(sa[dest[t, j]], s[t])
    live = np.zeros(M, dtype=bool)
    live[dest[dest >= 0]] = True
    assert written.all() and not np.any(qa[~live]) and np.all(sa[~live] == 1.0)
    # rows beyond M are dropped, not wrapped
    dest2, _, _, _ = permute.quantize_permute(x, ids, offs, 100)
    assert np.all(dest2 < 100) and np.sum(dest2 >= 0) == np.sum((dest >= 0) & (dest < 100))
