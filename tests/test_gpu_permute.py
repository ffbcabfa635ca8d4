"""GPU parity of the quantise-and-permute step (route counts, tile layout, row permutation and
e4m3 1x128 quantisation) against the CPU oracle: integer and byte outputs must match exactly,
scales bit for bit."""

import numpy as np
import pytest
import torch

import mx_grouped_gemm_amd as bsg
from oracle import formats, gemm as og, permute as op
from tests.parity import say
from workloads.generate import MOE32, activations, routing_counts, routing_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(x, ids, E, T_tiles):
    """GPU path: counts -> tile layout -> permute + quantise, outputs pre-poisoned."""
    xd, idd = x.cuda(), torch.from_numpy(ids).cuda()
    counts = bsg.bsgemm_route_counts(idd, E)
    eo, _, _ = bsg.bsgemm_build_tiles(counts, T_tiles, padded=True)
    M = 128 * T_tiles
    qa = torch.full((M, x.shape[1]), 0xAB, dtype=torch.uint8, device="cuda")
    sa = torch.full((M, x.shape[1] // 128), float("nan"), dtype=torch.float32, device="cuda")
    dest = torch.full(ids.shape, -7, dtype=torch.int32, device="cuda")
    bsg.bsgemm_quantize_permute(xd, idd, eo, M, E, dest=dest, qa=qa, a_scales=sa)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), eo.cpu().numpy(), dest.cpu().numpy(), qa.cpu().numpy(), sa.cpu().numpy()


def _check(x, ids, E, T_tiles, label, rows=None):
    counts, eo, dest, qa, sa = _run(x, ids, E, T_tiles)
    M = 128 * T_tiles
    assert np.array_equal(counts, op.route_counts(ids, E)), f"{label}: counts"
    eo_ref, _, _ = og.tile_map(op.route_counts(ids, E), T_tiles)
    assert np.array_equal(eo, eo_ref), f"{label}: expert offsets"
    xf = x.float().numpy()
    dest_ref, qa_ref, sa_ref, written = op.quantize_permute(xf, ids, eo_ref, M)
    assert np.array_equal(dest, dest_ref), f"{label}: dest"
    sel = np.arange(M) if rows is None else rows
    w = written[sel]
    assert np.array_equal(qa[sel][w], qa_ref[sel][w]), f"{label}: qa bytes"
    assert np.array_equal(sa[sel][w].view(np.uint32), sa_ref[sel][w].view(np.uint32)), f"{label}: scales"
    assert np.all(qa[sel][~w] == 0xAB) and np.all(np.isnan(sa[sel][~w])), f"{label}: rows outside the groups"
    say(f"[permute] {label}: M={M} rows checked={len(sel)} written={int(w.sum())}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_small_ragged_routing(dtype):
    rng = np.random.default_rng(3)
    T, k, E, K = 300, 3, 7, 384
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[4, 2] = -1
    ids[17, 0] = E + 3                                       # dropped: outside the experts
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(dtype)
    x[5, 128:256] = 0                                        # an all-zero block
    x[6] *= 1e-20                                            # tiny values
    counts = op.route_counts(ids, E)
    T_tiles = int(sum(-(-c // 128) for c in counts)) + 1     # one spare tile past the groups
    _check(x, ids, E, T_tiles, f"small {dtype}")


def test_ties_subnormals_and_signed_zero():
    """Blocks whose max is 448 have scale exactly 1, so x / s is x itself: exact midpoints of
    the e4m3 grid must go to even codes, subnormals and -0.0 must encode as in the oracle."""
    pos = np.array([c for c in range(0x7F)], dtype=np.uint8)
    vals = formats.decode_e4m3fn(pos)
    mids = (vals[:-1] + vals[1:]) / 2
    pool = np.concatenate([mids, -mids, vals, -vals, [0.0, -0.0, 2.0 ** -11, -2.0 ** -12]])
    rng = np.random.default_rng(4)
    T, K, E = 16, 512, 2
    x = rng.choice(pool, size=(T, K)).astype(np.float32)
    x[:, ::128] = 448.0                                      # every block: amax 448, s = 1
    ids = np.stack([np.arange(E) for _ in range(T)]).astype(np.int32)
    _check(torch.from_numpy(x), ids, E, 2, "ties")


def test_moe32_full_size_sampled():
    """16384 tokens x top-8 over 32 experts (two empty), K = 7168 bf16: the gate_up input.
    dest and counts in full; qa and scales on the rows of 512 sampled tokens and every padding
    row."""
    counts = routing_counts(seed=0, **MOE32)
    T, k, E, K = MOE32["tokens"], MOE32["top_k"], MOE32["experts"], 7168
    ids = routing_topk(counts, T, k)
    x = activations(T, K)
    T_tiles = int(sum(-(-int(c) // 128) for c in counts))
    got = _run(x, ids, E, T_tiles)
    c_gpu, eo, dest, qa, sa = got
    assert np.array_equal(c_gpu, counts)
    eo_ref, _, _ = og.tile_map(counts, T_tiles)
    assert np.array_equal(eo, eo_ref)
    assert np.array_equal(dest, op.permute_dest(ids, eo_ref, 128 * T_tiles))
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(T, 512, replace=False))
    q, s = op.quantize_rows(x[toks].float().numpy())
    for n, t in enumerate(toks):
        for r in dest[t]:
            assert np.array_equal(qa[r], q[n]) and np.array_equal(sa[r].view(np.uint32), s[n].view(np.uint32))
    for e in range(E):
        lo, hi = eo_ref[e] + counts[e], eo_ref[e + 1]
        assert not np.any(qa[lo:hi]) and np.all(sa[lo:hi] == 1.0)
    say(f"[permute] moe32 full size: {len(toks)} tokens x {k} rows and all padding rows match")


@pytest.mark.parametrize("T,k,E,K,dtype", [(97, 10, 16, 128, torch.float32),
                                            (64, 3, 4096, 256, torch.bfloat16),
                                            (50, 1, 1, 256, torch.bfloat16)])
def test_edge_shapes(T, k, E, K, dtype):
    """top_k above 8 (the quantiser's destinations come in groups of 8), one K block, the
    largest expert count (a 16 KiB LDS histogram; most of the 4096 experts stay empty), and a
    single expert (its 78 padding rows shared by the 256 workgroups that rank it)."""
    rng = np.random.default_rng(T + k)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(dtype)
    counts = op.route_counts(ids, E)
    T_tiles = int(sum(-(-c // 128) for c in counts))
    _check(x, ids, E, T_tiles, f"edge T={T} k={k} E={E} K={K}")
