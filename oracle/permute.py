"""Activation quantisation and token permutation into the grouped GEMM's A (oracle; test
infrastructure, see the package docstring).

The grouped GEMM of the Modular MAX page "promote_accumulators" (section Args) takes A with its
rows grouped by expert (``expert_ids`` maps each group of rows to its expert) and a per-row,
per-128-K fp32 scale ``a_scales``. This module computes that input from token activations and a
top-k routing, by its plain definition:

* ``route_counts`` - rows each expert receives (one per token that picked it).
* ``permute_dest`` - the A row of every (token, slot) pick: expert e's picks fill rows
  ``expert_offsets[e] ..`` in token order (a reading: the pages do not order rows within a
  group; token order makes the layout unique).
* ``quantize_rows`` - 1 x 128 block quantisation to e4m3fn: ``s = amax / 448`` and
  ``q = rne_e4m3(clamp(x / s, -448, 448))``, both divisions in fp32 (amax 0 gives s = 1,
  q = 0), the per-block scaling the pages' FP8 operands carry (1 x 128 for A).
* ``encode_e4m3fn`` - round-to-nearest-even onto the e4m3fn grid (the OFP8 bit layout given
  in ``formats``), computed exactly in fp64 from the fp32 value.
* ``quantize_permute`` - the three together; padding rows of each group are zero with scale 1.

Pins: ``tests/test_oracle_permute.py`` (exhaustive code round trip, ties to even at every
midpoint, torch's own e4m3fn conversion, power-of-two invariance, permutation validity).
"""

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def encode_e4m3fn(values):
    """fp32-representable values with |v| <= 448 -> uint8 e4m3fn codes, round half to even.

    Subnormals are multiples of 2**-9 below 2**-6; normals carry a 3-bit mantissa. The sign
    bit follows the value's sign bit (so -0.0 and negatives that round to zero give 0x80).
    """
    v = np.asarray(values, dtype=np.float64)
    if np.any(np.isnan(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("encode_e4m3fn takes finite values with |v| <= 448")
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    codes = np.zeros(v.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: units of 2**-9; a result of 8 units is the smallest normal (code 0x08)
    codes[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        m, e = np.frexp(a[nrm])                  # a = m * 2**e, m in [0.5, 1)
        e = e - 1                                # a = (2m) * 2**e, 2m in [1, 2)
        mant = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)
        carry = mant == 8
        e = e + carry
        mant = np.where(carry, 0, mant)
        codes[nrm] = ((e + 7) << 3) | mant
    return (codes | (sign << 7)).astype(np.uint8)


def quantize_rows(x):
    """Rows of ``x`` (fp32 values, [R, K], K a multiple of 128) -> (q uint8 [R, K],
    s float32 [R, K/128])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    xb = x.reshape(R, K // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (xb / s[:, :, None]).astype(np.float32)                  # fp32 division, as defined
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_e4m3fn(y).reshape(R, K), s


def route_counts(topk_ids, num_experts):
    """Picks per expert; ids outside [0, num_experts) are not counted."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    ok = (ids >= 0) & (ids < num_experts)
    return np.bincount(ids[ok], minlength=num_experts)[:num_experts].astype(np.int32)


def permute_dest(topk_ids, expert_offsets, M):
    """A row of each pick ``topk_ids[t, j]`` (-1 for ids outside the experts or rows >= M)."""
    ids = np.asarray(topk_ids).astype(np.int64)
    T, k = ids.shape
    E = len(expert_offsets) - 1
    dest = np.full((T, k), -1, dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if 0 <= e < E:
                r = expert_offsets[e] + seen[e]
                seen[e] += 1
                if r < M:
                    dest[t, j] = r
    return dest.astype(np.int32)


def quantize_permute(x, topk_ids, expert_offsets, M):
    """(dest [T, k] int32, qa uint8 [M, K], a_scales float32 [M, K/128], written [M] bool).

    Row ``dest[t, j]`` of qa / a_scales holds the quantised token row ``x[t]``. The padding
    rows of each expert's group (after its picks, up to ``expert_offsets[e + 1]``) hold zero
    codes with scale 1. ``written`` marks the rows the operation defines; others are untouched.
    """
    x = np.asarray(x, dtype=np.float32)
    T, K = x.shape
    E = len(expert_offsets) - 1
    q, s = quantize_rows(x)
    dest = permute_dest(topk_ids, expert_offsets, M)
    counts = route_counts(topk_ids, E)
    qa = np.zeros((M, K), dtype=np.uint8)
    a_scales = np.zeros((M, K // BLOCK), dtype=np.float32)
    written = np.zeros(M, dtype=bool)
    for e in range(E):
        lo = min(expert_offsets[e] + counts[e], M)
        hi = min(expert_offsets[e + 1], M)
        a_scales[lo:hi] = 1.0
        written[lo:hi] = True
    for t in range(T):
        for j in range(dest.shape[1]):
            r = dest[t, j]
            if r >= 0:
                qa[r] = q[t]
                a_scales[r] = s[t]
                written[r] = True
    return dest, qa, a_scales, written
