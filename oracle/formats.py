"""Exact fp64 decoders for the element and scale formats (oracle; test infrastructure).

Formats are the ones the Triton Gluon page "Overlapping Accumulator
Block-Scaled Matrix Multiplication" names: ``float8_e4m3fn`` elements
(``random_quantized_tensor``), e2m1 elements stored two per ``uint8`` along K
(``to_packed_tensor(dim=1)``), and uint8 e8m0 scales (``MXScaleTensor``,
one per ``VEC_SIZE = 32`` K-elements). The pages give names, not bit layouts;
the layouts below are the OCP definitions (OFP8 e4m3fn, OCP MX v1.0 e2m1 and
e8m0):

* e4m3fn: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. No
  infinities; S.1111.111 is NaN; exponent 0 is subnormal ``m * 2**-9``.
* e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
  subnormal ``m * 0.5``. Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
* e8m0: ``2**(x - 127)``; ``x = 255`` is NaN; no zero.

Packing reading (the pages do not fix it): the low nibble of a byte holds the
even K index, the high nibble the odd one.
"""

import numpy as np


def decode_e4m3fn(codes):
    """uint8 codes (any shape) -> float64 values, exactly."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.ldexp(1.0, exp - 7)
    subnormal = man * np.ldexp(1.0, -9)
    val = np.where(exp == 0, subnormal, normal)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


def decode_e2m1(nibbles):
    """4-bit codes (values 0..15, any integer dtype) -> float64 values, exactly."""
    c = np.asarray(nibbles).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("e2m1 codes must be in [0, 15]")
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    exp = (c >> 1) & 0x3
    man = c & 0x1
    normal = (1.0 + man / 2.0) * np.ldexp(1.0, exp - 1)
    subnormal = man * 0.5
    return sign * np.where(exp == 0, subnormal, normal)


def unpack_e2m1(packed):
    """uint8 [..., K/2] holding two e2m1 codes per byte -> int codes [..., K].

    Element 2j is the low nibble of byte j, element 2j+1 the high nibble.
    """
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def decode_e8m0(codes):
    """uint8 scale codes -> float64 ``2**(code - 127)``; code 255 -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    val = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, val)


def decode_elements(q, fmt):
    """Decode an element array in format ``fmt`` ('e4m3' or 'e2m1').

    e4m3: ``q`` is uint8 [..., K]; e2m1: ``q`` is packed uint8 [..., K/2].
    """
    if fmt == "e4m3":
        return decode_e4m3fn(q)
    if fmt == "e2m1":
        return decode_e2m1(unpack_e2m1(q))
    raise ValueError(f"unknown element format {fmt!r}")
