"""GPU parity of the nvfp4 GEMM (e2m1 elements, one e4m3 scale per 16 K-elements) through the
C ABI, against the fp64 CPU oracle (``oracle.gemm.nv_gemm``).

Inputs come from the seeded generators in ``workloads`` (or are drawn here from a seeded torch
generator); expected values come only from the oracle.
"""

import numpy as np
import pytest
import torch

import mx_grouped_gemm_amd as bsg
from oracle import gemm as og
from tests.parity import check, gpu_tile_map, poisoned, run_problem, sample_rows, say
from workloads.generate import make_problem, nv_problem

pytestmark = pytest.mark.gpu

GPU = torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not GPU:
        pytest.skip("no GPU")
    say(f"\n[gpu-test] {request.node.name}")


def _run(qa, sa, qb, sb, M, N, K, out, ei=None, to=None, E=1):
    C = poisoned(M, N, out)
    bsg.bsgemm_grouped(qa, sa, qb, sb, ei, to, C, M, N, K, bsg.make_fmt("e2m1", "e2m1", "nv", out),
                       num_tiles=None if ei is None else ei.numel(), num_experts=E)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("out", ["f16", "bf16", "f32"])
def test_nv_dense_ragged(out):
    """320 rows (two super-tiles, the second a lone 64-row tile), N = 384 (a 128-column tail),
    K = 512 (two stages)."""
    p = nv_problem(320, 384, 512, device="cuda", seed=41)
    C, _, _ = run_problem(p, out)
    check(p, out, C, label="nvfp4 320x384x512")


@pytest.mark.parametrize("K", [256, 768, 2048])
def test_nv_k_depths(K):
    p = nv_problem(256, 256, K, device="cuda", seed=K + 1)
    C, _, _ = run_problem(p, "f32")
    check(p, "f32", C, label=f"nvfp4 K={K}")


def test_nv_exact_products_bit_exact():
    """Layout pin for codes, nibbles and the per-16 scales: scales 1 .. 1.875 (every mantissa)
    and K = 256 keep every partial sum exact in fp32, so the output must equal the oracle bit
    for bit; a scale taken from the wrong 16-block or row changes the exact value."""
    g = torch.Generator(device="cpu").manual_seed(43)
    M, N, K = 128, 256, 256
    qa = torch.randint(0, 256, (M, K // 2), generator=g, dtype=torch.uint8)
    qb = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
    sa = torch.randint(0x38, 0x40, (M, K // 16), generator=g, dtype=torch.uint8)
    sb = torch.randint(0x38, 0x40, (N, K // 16), generator=g, dtype=torch.uint8)
    C = _run(qa.cuda(), sa.cuda(), qb[None].cuda(), sb[None].cuda(), M, N, K, "f32")
    ref = og.nv_gemm(qa.numpy(), sa.numpy(), qb.numpy(), sb.numpy())
    got = C.cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != ref)
    say(f"[nv-exact] mismatches={len(bad)}")
    assert len(bad) == 0, f"first mismatches at {bad[:5].tolist()}"


def test_nv_every_scale_code():
    """Scale codes over the whole finite e4m3 range (subnormal, negative, 448) on both operands:
    every scaled element is still exact in f16, so only fp32 summation differs."""
    g = torch.Generator(device="cpu").manual_seed(44)
    M, N, K = 256, 256, 512
    qa = torch.randint(0, 256, (M, K // 2), generator=g, dtype=torch.uint8)
    qb = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)

    def codes(shape):
        c = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
        return torch.where((c & 0x7F) == 0x7F, c ^ 1, c)           # no NaN codes

    sa, sb = codes((M, K // 16)), codes((N, K // 16))
    C = _run(qa.cuda(), sa.cuda(), qb[None].cuda(), sb[None].cuda(), M, N, K, "f32")
    ref = og.nv_gemm(qa.numpy(), sa.numpy(), qb.numpy(), sb.numpy())
    den = og.nv_gemm(qa.numpy(), sa.numpy(), qb.numpy(), sb.numpy(), absolute=True)
    err = og.relative_error(C.cpu().numpy(), ref, den)
    say(f"[nv-codes] max_rel_err={err:.3e}")
    assert err <= 1e-3


def test_nv_grouped_tile_map():
    """Grouped through the GPU tile map: a ragged group, an empty expert, a group of 7 rows."""
    p = nv_problem(0, 256, 512, device="cuda", seed=45, counts=[130, 0, 100, 7])
    C, _, _ = run_problem(p, "bf16")
    check(p, "bf16", C, label="nvfp4 grouped")


def test_nv_grouped_compact_layout():
    """The packed (unpadded) tile map: groups back to back, ragged last tiles."""
    counts = [70, 200, 0, 33]
    M, N, K = int(sum(counts)), 256, 256
    p = nv_problem(M, N, K, device="cuda", seed=46)
    qb = torch.cat([p.qb] + [nv_problem(8, N, K, device="cuda", seed=47 + e).qb for e in range(3)])
    sb = torch.cat([p.b_scales] + [nv_problem(8, N, K, device="cuda", seed=47 + e).b_scales
                                   for e in range(3)])
    T = sum(-(-c // 128) for c in counts)
    _, to, ei = gpu_tile_map(counts, T, padded=False)
    C = _run(p.qa, p.a_scales, qb.contiguous(), sb.contiguous(), M, N, K, "f16", ei, to, E=4)
    _, to_r, ei_r = og.tile_map(counts, T, padded=False)
    assert np.array_equal(ei.cpu().numpy(), ei_r)
    args = [t.cpu().numpy() for t in (p.qa, p.a_scales, qb, sb)]
    ref = og.nv_gemm(*args, ei_r, to_r)
    den = og.nv_gemm(*args, ei_r, to_r, absolute=True)
    err = og.relative_error(C.float().cpu().numpy(), ref, den)
    say(f"[nv-compact] max_rel_err={err:.3e}")
    assert err <= 1e-3


def test_nvfp4_8192_sampled():
    """The benchmarked workload (8192^3, fp16 out) at full size, checked on sampled rows."""
    p = make_problem("nvfp4_8192", device="cuda")
    C, _, _ = run_problem(p, "f16")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(C).all()), "non-finite output"
    check(p, "f16", C, rows=sample_rows(p), label="nvfp4_8192")
    del C, p
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K", [512, 1024, 2048, 4096])
def test_nv_k_sweep(K):
    """The K values of the pages' benchmark sweep (M = N = 1024 here so the oracle is quick)."""
    p = nv_problem(1024, 1024, K, device="cuda", seed=K + 7)
    C, _, _ = run_problem(p, "f16")
    check(p, "f16", C, rows=sample_rows(p, seed=K), label=f"nvfp4 sweep K={K}")


def test_nv_skipped_and_out_of_range_tiles():
    """Tiles with id -1 or an id >= num_experts are skipped: their rows keep the poison."""
    p = nv_problem(0, 256, 512, device="cuda", seed=48, counts=[128, 128])
    ei = torch.tensor([1, -1, 0, 9], dtype=torch.int32, device="cuda")
    to = torch.tensor([0, 128, 256, 384, 512], dtype=torch.int32, device="cuda")
    M = 512
    qa = torch.cat([p.qa, torch.zeros(M - p.M, p.K // 2, dtype=torch.uint8, device="cuda")])
    sa = torch.cat([p.a_scales, torch.full((M - p.M, p.K // 16), 0x38, dtype=torch.uint8, device="cuda")])
    C = _run(qa, sa, p.qb, p.b_scales, M, p.N, p.K, "f32", ei, to, E=2)
    assert torch.all(torch.isnan(C[128:256])) and torch.all(torch.isnan(C[384:]))
    args = [t.cpu().numpy() for t in (qa, sa, p.qb, p.b_scales)]
    ei_r, to_r = np.array([1, -1, 0, -1]), to.cpu().numpy()
    ref = og.nv_gemm(*args, ei_r, to_r)
    den = og.nv_gemm(*args, ei_r, to_r, absolute=True)
    live = np.r_[0:128, 256:384]
    err = og.relative_error(C.cpu().numpy()[live], ref[live], den[live])
    say(f"[nv-skip] max_rel_err={err:.3e}")
    assert err <= 1e-3


def test_nv_deterministic():
    """Two runs of the same nvfp4 launch give the same bits."""
    p = nv_problem(640, 512, 1024, device="cuda", seed=49)
    C1, _, _ = run_problem(p, "f16")
    C2, _, _ = run_problem(p, "f16")
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
