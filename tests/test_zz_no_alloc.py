"""The entry point that allocates nothing (bsgemm_grouped_noalloc) against the workspace one
(bsgemm_grouped_ws), through the C ABI: two calls in a row, the second smaller, each compared
with the fp64 oracle at the tolerance of every blockwise parity test and with the workspace
entry point's output (same relative metric; with at most 64 partial tiles the no-alloc call may
cut items into fewer K ranges, so the fp32 sums may round differently)."""

import numpy as np
import pytest
import torch

import mx_grouped_gemm_amd as bsg
from oracle import gemm as og
from tests.parity import TOL, check, poisoned, say
from workloads.generate import blockwise_problem

pytestmark = pytest.mark.gpu

GPU = torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not GPU:
        pytest.skip("no GPU")
    say(f"\n[gpu-test] {request.node.name}")


def both(p, out, ws):
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", out)
    C_ws, C_na = poisoned(p.M, p.N, out), poisoned(p.M, p.N, out)
    bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C_ws, p.M, p.N, p.K, fmt, ws)
    bsg.bsgemm_grouped_noalloc(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C_na, p.M, p.N, p.K, fmt)
    torch.cuda.synchronize()
    return C_ws, C_na


def test_noalloc_matches_workspace_entry_two_calls():
    ws = torch.empty(bsg.bsgemm_grouped_workspace_size(), dtype=torch.uint8, device="cuda")
    # first call: 8 items of a long K (the split applies: 8 ranges here, 16 with a full workspace);
    # second, smaller: 2 items, 4 ranges
    for label, (M, N, K, out) in (("call 1", (256, 2048, 16384, "f32")), ("call 2", (128, 512, 4096, "bf16"))):
        p = blockwise_problem(None, N, K, device="cuda", a_rows=M, seed=M + N + K)
        C_ws, C_na = both(p, out, ws)
        check(p, out, C_na, label=f"no-alloc {label}")
        qa, sa, qb, sb = (t.cpu().numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales))
        den = og.blockwise_grouped_dequant(qa, sa, qb, sb, absolute=True)
        err = og.relative_error(C_na.float().cpu().numpy().astype(np.float64),
                                C_ws.float().cpu().numpy().astype(np.float64), den)
        say(f"[no-alloc] {label}: vs workspace entry point max_rel_err={err:.3e}")
        assert err <= TOL[out]


def test_noalloc_dynamic_work_order_bit_identical():
    """Whole items of 40 K blocks or more (8192 x 2048 x 5120: 256 items): the no-alloc call takes
    each XCD's items from counters in the library's scratch; two calls in a row, each equal bit for
    bit to bsgemm_grouped (same per-item arithmetic)."""
    p = blockwise_problem(None, 2048, 5120, device="cuda", a_rows=8192, seed=61)
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16")
    C_ref = poisoned(p.M, p.N, "bf16")
    bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C_ref, p.M, p.N, p.K, fmt)
    for call in (1, 2):
        C = poisoned(p.M, p.N, "bf16")
        bsg.bsgemm_grouped_noalloc(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C, p.M, p.N, p.K, fmt)
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), C_ref.view(torch.int16)), f"call {call}"
        say(f"[no-alloc] dynamic order call {call}: bit-identical")


def test_noalloc_last_round_split_matches_workspace_call():
    """8448 x 2048 x 4096 (264 items): the last 8 items are cut into 8 K ranges whose partial tiles
    fit the library's scratch as they fit a full workspace, so the no-alloc call equals the
    workspace call bit for bit, twice in a row, and bsgemm_grouped outside those items."""
    p = blockwise_problem(None, 2048, 4096, device="cuda", a_rows=8448, seed=62)
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16")
    ws = torch.empty(bsg.bsgemm_grouped_workspace_size(), dtype=torch.uint8, device="cuda")
    C_ws = poisoned(p.M, p.N, "bf16")
    bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C_ws, p.M, p.N, p.K, fmt, ws)
    C_ref = poisoned(p.M, p.N, "bf16")
    bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C_ref, p.M, p.N, p.K, fmt)
    torch.cuda.synchronize()
    assert torch.equal(C_ws[:8192].view(torch.int16), C_ref[:8192].view(torch.int16))
    for call in (1, 2):
        C = poisoned(p.M, p.N, "bf16")
        bsg.bsgemm_grouped_noalloc(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C, p.M, p.N, p.K, fmt)
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), C_ws.view(torch.int16)), f"call {call}"
    check(p, "bf16", C, rows=np.arange(8192, 8448), label="no-alloc last-round split")
