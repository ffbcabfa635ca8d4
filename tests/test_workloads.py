"""Checks of the seeded workload generator (CPU only)."""

import numpy as np
import torch

from workloads.generate import (MOE8, MOE32, blockwise_problem, make_problem, padded_starts,
                                routing_counts)


def test_routing_counts_rules():
    c8 = routing_counts(seed=0, **MOE8)
    assert c8.sum() == 4096 * 2 and c8.max() <= 4096 and len(c8) == 8
    c32 = routing_counts(seed=0, **MOE32)
    assert c32.sum() == 16384 * 8 and c32.max() <= 16384 and len(c32) == 32
    assert np.sum(c32 == 0) >= 2                       # the forced-empty experts
    assert np.array_equal(c32, routing_counts(seed=0, **MOE32))   # seeded


def test_padded_layout():
    counts = np.array([3, 0, 130, 128])
    assert padded_starts(counts).tolist() == [0, 128, 128, 384, 512]
    p = blockwise_problem(counts, 128, 256, seed=1)
    assert p.M == 512 and p.E == 4
    assert p.qa.shape == (512, 256) and p.a_scales.shape == (512, 2)
    assert p.qb.shape == (4, 128, 256) and p.b_scales.shape == (4, 1, 2)
    # padding rows: zero codes, unit scales
    assert torch.all(p.qa[3:128] == 0) and torch.all(p.a_scales[3:128] == 1)
    assert torch.all(p.qa[258:384] == 0)
    assert p.real_rows == 261


def test_config0_and_outliers():
    p = make_problem("single_128x256x512")
    assert (p.M, p.N, p.K, p.E) == (128, 256, 512, 1) and p.out_dtypes == ("f32", "bf16")
    # no NaN codes are ever produced
    for q in (p.qa, p.qb):
        assert not torch.any((q == 0x7F) | (q == 0xFF))
    assert torch.all(p.a_scales > 0) and torch.all(p.b_scales > 0)


def test_outlier_rows_move_scales():
    p = blockwise_problem(None, 128, 256, a_rows=128, seed=0, outlier_every=64)
    s = p.a_scales
    assert torch.all(s[0] > 20 * s[1]) and torch.all(s[64] > 20 * s[65])
