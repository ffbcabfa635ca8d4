"""Pins for the oracle's format decoders (CPU only).

Each decoder is checked against values the format specifications print
(``tests/golden``) and, where torch has the type, against torch's own
conversion to float32 over every code.
"""

import math

import numpy as np
import pytest
import torch

from oracle import formats
from workloads.generate import _e2m1_codes, pack_e2m1, quantize_mx


def _val(s):
    return float(s)


def test_e4m3_golden_points(golden):
    for code, value in golden("ofp8_e4m3fn_points.txt"):
        got = float(formats.decode_e4m3fn(np.uint8(int(code, 16))))
        want = _val(value)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.decode_e4m3fn(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_e8m0_golden_and_torch(golden):
    for code, value in golden("mx_e8m0_points.txt"):
        got = float(formats.decode_e8m0(np.uint8(int(code))))
        want = _val(value)
        assert (math.isnan(got) and math.isnan(want)) or got == want, code
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().double().numpy()
    ours = formats.decode_e8m0(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])


def test_e2m1_golden(golden):
    rows = golden("mx_e2m1_values.txt")
    assert len(rows) == 16
    for code, value in rows:
        got = float(formats.decode_e2m1(int(code)))
        want = _val(value)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e2m1_packing_low_nibble_first():
    # byte 0x72: element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    packed = np.array([[0x72, 0x9F]], np.uint8)
    vals = formats.decode_elements(packed, "e2m1")
    assert vals.tolist() == [[1.0, 6.0, -6.0, -0.5]]


def test_generator_e2m1_encoder_roundtrip():
    """Encoding each representable value returns its code (the workload's encoder)."""
    codes = np.arange(16)
    vals = torch.tensor(formats.decode_e2m1(codes), dtype=torch.float32)
    enc = _e2m1_codes(vals).numpy()
    # -0.0 encodes as +0 (code 0); every other code is recovered
    assert np.array_equal(enc[codes != 8], codes[codes != 8])


def test_generator_e2m1_encoder_ties_to_even():
    x = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, 0.26, 2.51])
    got = formats.decode_e2m1(_e2m1_codes(x).numpy()).tolist()
    assert got == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.5, 3.0]


def test_generator_mx_scale_rule():
    """e8m0 code = floor(log2 amax) - emax + 127, from frexp (exact at powers of two)."""
    x = torch.zeros(1, 64)
    x[0, 0] = 448.0     # block 0: amax = 448 -> floor(log2) = 8 -> e4m3 code 127 + 8 - 8
    x[0, 32] = 1.0      # block 1: amax = 1 -> code 127 - 8
    q, s = quantize_mx(x, "e4m3")
    assert s.tolist() == [[127, 119]]
    deq = formats.decode_e4m3fn(q.numpy()) * np.repeat(formats.decode_e8m0(s.numpy()), 32, axis=1)
    assert deq[0, 0] == 448.0 and deq[0, 32] == 1.0
    q4, s4 = quantize_mx(x, "e2m1")
    assert s4.tolist() == [[133, 125]]
    deq4 = formats.decode_elements(q4.numpy(), "e2m1") * np.repeat(formats.decode_e8m0(s4.numpy()), 32, axis=1)
    # 448 * 2**-6 = 7 saturates to 6 (e2m1 max), so the block's max decodes to 384
    assert deq4[0, 0] == 384.0 and deq4[0, 32] == 1.0


def test_pack_matches_unpack():
    codes = torch.randint(0, 16, (3, 64), generator=torch.Generator().manual_seed(1))
    packed = pack_e2m1(codes).numpy()
    assert np.array_equal(formats.unpack_e2m1(packed), codes.numpy())


def test_decoders_reject_bad_e2m1():
    with pytest.raises(ValueError):
        formats.decode_e2m1(16)
