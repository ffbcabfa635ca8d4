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


def tail_parts(tiles, N, K, slots=None):
    """Ranges per item of the last round's items in a whole-items launch through the workspace
    (the library's rule; 1: none)."""
    G = num_cus() // 8 * 8
    items, KB = items_of(tiles, N), K // 128
    if items < G or items >= 4 * G:
        return 1
    slots = G if slots is None else min(G, slots)
    last, t = items % G, 1
    while last > 0 and t < 16 and KB >= 2 * t * 4 and last * 2 * t <= slots and 16 + last * 2 * t < ERR_WORD:
        t *= 2
    return t


def item_cell(L, tiles, N):
    """(super-tile, first column) of work item L in the kernel's order: groups of group_m
    super-tiles (1 with at most 8 column blocks, else 4) walk their column blocks together."""
    n_blocks = -(-N // 256)
    group_m = 1 if n_blocks <= 8 else 4
    gsz = group_m * n_blocks
    g0 = (L // gsz) * group_m
    gm = min(group_m, (tiles + 1) // 2 - g0)
    r = L % gsz
    return g0 + r % gm, (r // gm) * 256


def tail_mask(p, tile_offsets=None):
    """Boolean [M, N] over the cells of the last round's items (rows of both tiles of the
    super-tile, by tile_offsets; padded layout when None)."""
    T = p.M // 128
    G = num_cus() // 8 * 8
    items = items_of(T, p.N)
    to = np.arange(T + 1) * 128 if tile_offsets is None else tile_offsets.cpu().numpy()
    mask = np.zeros((p.M, p.N), bool)
    for L in range(items - items % G, items):
        s, n0 = item_cell(L, T, p.N)
        for t in (2 * s, 2 * s + 1):
            if t < T:
                r0 = int(to[t])
                mask[r0:r0 + min(128, int(to[t + 1]) - r0), n0:n0 + 256] = True
    return torch.from_numpy(mask).cuda()


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
    asked again), their rows stay untouched. Outside the last round's items (cut along K into
    ranges, whose partial sums round differently) everything matches bsgemm_grouped bit for bit;
    two calls give the same bits."""
    rng = np.random.default_rng(11)
    counts = rng.integers(0, 4000, 40)
    counts[[2, 9]] = 0
    p = blockwise_problem([int(c) for c in counts], 256, 5120, device="cuda", seed=52)
    T = p.M // 128
    assert _dyn_applies(T, p.N, p.K)
    say(f"[dyn] items={items_of(T, p.N)} last-round ranges per item={tail_parts(T, p.N, p.K)}")
    _, to, ei = gpu_tile_map(p.counts, T)
    ei = ei.clone()
    ei.view(-1)[0::8] = 1000     # both tiles of every fourth super-tile: expert out of range
    ei.view(-1)[1::8] = -1
    C_static, outs = _static_and_ws(p, ei, to, "bf16", workspace)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    mask = tail_mask(p, to) if tail_parts(T, p.N, p.K) > 1 else torch.zeros_like(C_static, dtype=torch.bool)
    for C in outs:
        assert torch.equal(C.view(torch.int16)[~mask], C_static.view(torch.int16)[~mask])
    ei_h = ei.cpu().numpy().copy()
    ei_h[(ei_h < 0) | (ei_h >= p.E)] = -1
    check(p, "bf16", outs[-1], rows=sample_rows(p), tile_map_ref=(ei_h, to.cpu().numpy()),
          label="dynamic order with skipped items")


@pytest.mark.parametrize("M,N,K,out", [
    (8448, 2048, 4096, "bf16"),   # 264 items: 256 whole (static order), the last 8 in 8 ranges of 4
    (8704, 4096, 5120, "f32"),    # 544 items: dynamic order, the last 32 in 8 ranges of 5 blocks
    (16640, 2048, 4096, "f16"),   # 520 items: static order, the last 8 in 8 ranges of 4 blocks
])
def test_last_round_split_dense(workspace, M, N, K, out):
    """The last round's items, fewer than the grid, are cut along K and taken by the workgroups
    that finish first: the oracle on every row of those items and sampled rows elsewhere, the
    rest bit-identical to bsgemm_grouped, two calls bit-identical."""
    T = M // 128
    parts = tail_parts(T, N, K)
    say(f"[tail] items={items_of(T, N)} ranges per item={parts}")
    assert parts >= 2
    p = blockwise_problem(None, N, K, device="cuda", a_rows=M, seed=M + N)
    C_static, outs = _static_and_ws(p, None, None, out, workspace)
    assert int(workspace[: 4 * (ERR_WORD + 1)].view(torch.int32)[ERR_WORD]) == 0
    bits = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(outs[0].view(bits), outs[1].view(bits))
    mask = tail_mask(p)
    assert bool(mask.any())
    assert torch.equal(outs[0].view(bits)[~mask], C_static.view(bits)[~mask])
    tail_rows = np.nonzero(mask.any(dim=1).cpu().numpy())[0]
    rows = np.union1d(sample_rows(p, per_tile=10), tail_rows)
    check(p, out, outs[0], rows=rows, label=f"last-round split {M}x{N}x{K}")


def test_last_round_split_moe8(workspace):
    """The 8-expert workload (272 items, the last 16 in 8 ranges; tiles of two experts share
    super-tiles): oracle on sampled rows of every tile and on all rows of the last round's items."""
    from workloads.generate import make_problem
    p = make_problem("moe8_n2048_k4096", device="cuda", seed=0)
    T = p.M // 128
    parts = tail_parts(T, p.N, p.K)
    say(f"[tail] items={items_of(T, p.N)} ranges per item={parts}")
    assert parts >= 2
    _, to, ei = gpu_tile_map(p.counts, T)
    C_static, outs = _static_and_ws(p, ei, to, "bf16", workspace)
    assert int(workspace[: 4 * (ERR_WORD + 1)].view(torch.int32)[ERR_WORD]) == 0
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    mask = tail_mask(p, to)
    assert torch.equal(outs[0].view(torch.int16)[~mask], C_static.view(torch.int16)[~mask])
    tail_rows = np.nonzero(mask.any(dim=1).cpu().numpy())[0]
    rows = np.union1d(sample_rows(p, per_tile=4), tail_rows)
    check(p, "bf16", outs[0], rows=rows, label="last-round split moe8")
