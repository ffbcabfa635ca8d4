"""GPU parity of the split-K schedule (bsgemm_grouped_ws): a problem with fewer 256 x 256 work
items than compute units has each item cut along K into 2-16 ranges run side by side; the ranges'
fp32 partial tiles are summed into C, each range reducing a slice of the tile.

Every case is small enough that the split launch runs (checked here with the same rule the
library applies); results are compared with the fp64 oracle at the same tolerance as
bsgemm_grouped. The workspace's error word (set only if a workgroup ever gave up waiting for
the other ranges of its item) must stay zero, and calls in a row on one workspace check that the
flags are cleared between calls.
"""

import numpy as np
import pytest
import torch

import mx_grouped_gemm_amd as bsg
from tests.parity import check, gpu_tile_map, poisoned, sample_rows, say
from workloads.generate import blockwise_problem

pytestmark = pytest.mark.gpu

GPU = torch.cuda.is_available()
ERR_WORD = 1023   # int32 index of the error word in the workspace's first 4 KiB


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not GPU:
        pytest.skip("no GPU")
    say(f"\n[gpu-test] {request.node.name}")


@pytest.fixture(scope="module")
def workspace():
    n = bsg.bsgemm_grouped_workspace_size()
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def num_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def items_of(tiles, N):
    return -(-tiles // 2) * (N // 256)


def split_parts(tiles, N, K):
    """K ranges per item under the library's rule (1: no split)."""
    G = num_cus() // 8 * 8
    items, KB, parts = items_of(tiles, N), K // 128, 1
    if items >= G:
        return 1
    while parts < 16 and 2 * parts * 8 <= KB and items * 2 * parts <= G:
        parts *= 2
    return parts


def run_ws(p, out, ws, tile_map=None):
    C = poisoned(p.M, p.N, out)
    ei = to = None
    if p.counts is not None:
        _, to, ei = gpu_tile_map(p.counts, p.M // 128)
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", out)
    bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, ei, to, C, p.M, p.N, p.K, fmt, ws,
                          num_tiles=None if ei is None else ei.numel(), num_experts=p.E)
    torch.cuda.synchronize()
    assert int(ws[: 4 * (ERR_WORD + 1)].view(torch.int32)[ERR_WORD]) == 0, "a split range timed out"
    return C


def test_workspace_size_and_errors(workspace):
    G = num_cus() // 8 * 8
    assert workspace.numel() == 4096 + G * 256 * 256 * 4
    p = blockwise_problem(None, 256, 2048, device="cuda", a_rows=256, seed=1)
    C = poisoned(p.M, p.N, "f32")
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "f32")
    small = workspace[: workspace.numel() - 1]
    with pytest.raises(bsg.BsgemmError) as e:
        bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C, p.M, p.N, p.K, fmt, small)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert bool(torch.isnan(C).all())


@pytest.mark.parametrize("M,N,K,out", [
    (256, 2048, 16384, "f32"),    # 8 items, 16 ranges of 8 blocks
    (1000, 4096, 2048, "bf16"),   # 64 items (ragged last tile), 2 ranges
    (200, 1024, 2304, "f32"),     # 4 items, 2 ranges of 9 blocks (odd: chunk boundary inside)
    (384, 768, 5120, "f16"),      # 6 items (one super-tile of a lone 128-row tile), 4 ranges of 10
])
def test_dense_split(workspace, M, N, K, out):
    assert split_parts(-(-M // 128), N, K) >= 2
    p = blockwise_problem(None, N, K, device="cuda", a_rows=M, seed=M + K)
    C = run_ws(p, out, workspace)
    check(p, out, C, label=f"split dense {M}x{N}x{K}")


@pytest.mark.parametrize("counts,N,K", [
    ([100, 300, 0, 50], 1024, 4096),     # two-pass items (tiles of different experts), an empty expert
    ([129, 1, 0, 256, 7], 512, 8192),    # ragged groups padded to 128, 16 ranges
])
def test_grouped_split(workspace, counts, N, K):
    p = blockwise_problem(counts, N, K, device="cuda", seed=K + len(counts))
    parts = split_parts(p.M // 128, N, K)
    say(f"[split] items={items_of(p.M // 128, N)} ranges per item={parts}")
    assert parts >= 2
    C = run_ws(p, "bf16", workspace)
    check(p, "bf16", C, label=f"split grouped {counts}")


def test_two_calls_second_smaller(workspace):
    """Two calls in a row on one workspace, the second smaller: flags cleared in between."""
    assert split_parts(4, 4096, 4096) >= 2 and split_parts(2, 1024, 2048) >= 2
    p1 = blockwise_problem(None, 4096, 4096, device="cuda", a_rows=512, seed=31)
    p2 = blockwise_problem(None, 1024, 2048, device="cuda", a_rows=256, seed=32)
    C1 = run_ws(p1, "bf16", workspace)
    C2 = run_ws(p2, "bf16", workspace)
    check(p1, "bf16", C1, label="split call 1")
    check(p2, "bf16", C2, label="split call 2")


def test_large_problem_runs_whole_items(workspace):
    """With at least as many items as compute units the call is bsgemm_grouped's (bit-identical)."""
    p = blockwise_problem(None, 4096, 512, device="cuda", a_rows=8192, seed=33)
    C1 = run_ws(p, "bf16", workspace)
    C2 = poisoned(p.M, p.N, "bf16")
    bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C2, p.M, p.N, p.K,
                       bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16"))
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


def _dyn_applies(tiles, N, K):
    """The library's rule for the dynamic work order (whole items through the workspace)."""
    G = num_cus() // 8 * 8
    return items_of(tiles, N) >= G and K // 128 >= 40 and split_parts(tiles, N, K) == 1


def _static_and_ws(p, ei, to, out, ws, calls=2):
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", out)
    nt = None if ei is None else ei.numel()
    C_static = poisoned(p.M, p.N, out)
    bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, ei, to, C_static, p.M, p.N, p.K, fmt,
                       num_tiles=nt, num_experts=p.E)
    outs = []
    for _ in range(calls):   # calls in a row on one workspace: the counters are cleared each time
        C = poisoned(p.M, p.N, out)
        bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, ei, to, C, p.M, p.N, p.K, fmt, ws,
                              num_tiles=nt, num_experts=p.E)
        outs.append(C)
    torch.cuda.synchronize()
    return C_static, outs


def test_dynamic_work_order_dense_bit_identical(workspace):
    """8192 x 2048 x 5120 (256 items of 40 K blocks): the workspace call takes each XCD's items
    from a counter; every item is computed as in bsgemm_grouped, so the output is the same bit for
    bit (and within the oracle's tolerance on sampled rows)."""
    p = blockwise_problem(None, 2048, 5120, device="cuda", a_rows=8192, seed=51)
    assert _dyn_applies(p.M // 128, p.N, p.K)
    C_static, outs = _static_and_ws(p, None, None, "bf16", workspace)
    for C in outs:
        assert torch.equal(C.view(torch.int16), C_static.view(torch.int16))
    check(p, "bf16", outs[-1], rows=sample_rows(p), label="dynamic order dense")


def test_dynamic_work_order_grouped_with_skipped_items(workspace):
    """Ragged groups of 40 experts at K = 5120 with every fourth super-tile's tiles given an
    out-of-range expert id: items without a live tile are taken and passed over (the counter is
    asked again), their rows stay untouched, and everything matches bsgemm_grouped bit for bit."""
    rng = np.random.default_rng(11)
    counts = rng.integers(0, 4000, 40)
    counts[[2, 9]] = 0
    p = blockwise_problem([int(c) for c in counts], 256, 5120, device="cuda", seed=52)
    T = p.M // 128
    assert _dyn_applies(T, p.N, p.K)
    _, to, ei = gpu_tile_map(p.counts, T)
    ei = ei.clone()
    ei.view(-1)[0::8] = 1000     # both tiles of every fourth super-tile: expert out of range
    ei.view(-1)[1::8] = -1
    C_static, outs = _static_and_ws(p, ei, to, "bf16", workspace)
    for C in outs:
        assert torch.equal(C.view(torch.int16), C_static.view(torch.int16))
    ei_h = ei.cpu().numpy().copy()
    ei_h[(ei_h < 0) | (ei_h >= p.E)] = -1
    check(p, "bf16", outs[-1], rows=sample_rows(p), tile_map_ref=(ei_h, to.cpu().numpy()),
          label="dynamic order with skipped items")
