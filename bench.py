"""Benchmark: grouped blockwise-FP8 MoE GEMM on one MI355X.

One step = one pass of the hot path over one batch of the large MoE workload (32 local
experts, 16384 tokens at top-8 = 131072 expert rows, Dirichlet(1.0) routing with two empty
experts, padded to 128-row tiles):
    1. token-to-expert tile map from the per-expert counts (GPU kernel),
    2. gate_up grouped GEMM  N=4096, K=7168  (e4m3, 1x128 / 128x128 fp32 scales, bf16 out),
    3. down    grouped GEMM  N=7168, K=2048  (same formats).
Inputs are synthetic (seeded) and resident in HBM before the timed region. ``value`` is
useful TFLOP/s (2 * real rows * N * K summed over both GEMMs, padding rows excluded) per
step time. The JSON line also carries the roofline of the dominant kernel (gate_up), whose
per-launch time is measured with HIP events on the stream the kernels run on, and the CPU
oracle's rate on a bounded sample of the same workload.

With --workload mx8192_<a>_<b> a step is instead one dense MX GEMM of 8192^3 (e8m0 scales per
32 K, fp16 out) with formats a x b; its roofline is that launch against the peak of the
narrower-rate format pair.

With --workload nvfp4_8192 a step is one dense nvfp4 GEMM of 8192^3 (e2m1 elements, an e4m3
scale per 16 K, fp16 out); the products run on the f16 matrix instruction, so its roofline is
against the f16 peak.

With --workload dense_4096 (one group 4096^3, every 64th row of A and B x100), moe8_n2048_k4096
(8 experts, 4096 tokens at top-2, Dirichlet(0.5), N=2048, K=4096) or dense_256x2048x16384 (8 work
items with a long K) a step is the tile map (grouped only) and one blockwise-FP8 GEMM call, bf16
out, through bsgemm_grouped_ws (its split-K schedule applies to the last one only; --no-split
calls bsgemm_grouped); its roofline is that call against the FP8 peak.

With --workload permute_moe32 a step is the step before the GEMM on the same routing: per-expert
counts of the top-8 picks, the tile map, and the permutation of the 16384 bf16 token rows
(K = 7168) into the padded expert-sorted A with e4m3 1x128 quantisation. It is HBM-bound: the
value is GB/s of algorithmic bytes and the roofline is against the 8 TB/s HBM peak.

With --workload decode_moe32 a step is the gate_up GEMM (N=4096, K=7168, 32 experts) for a
decode batch of 128 tokens x top-8 (about 34 rows per expert), with the schedule for M-tiles of
few rows (fmt | SCHED_SMALL_M). Streaming B bounds it: GB/s of algorithmic bytes against the
HBM peak; the large-tile schedule is timed beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--workload W]
       python bench.py --copy-calibration MIB --steps K   (HBM counter calibration)
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5033.0   # MI355X dense FP8 MFMA peak (256 CU x 2.4 GHz x 8192 flop/clk)
PEAK_FP4_TFLOPS = 10066.0  # MI355X dense MXFP4 MFMA peak (twice the FP8 rate)
PEAK_FP16_TFLOPS = 2516.6  # MI355X dense FP16 MFMA peak (half the FP8 rate)
PEAK_HBM_GBS = 8000.0
METRIC = "TFLOP/s + % of MI355X FP8 dense peak, grouped blockwise-FP8 GEMM"

# HBM bytes per gate_up launch: rocprofv3 FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 (factors from a
# 1 GiB device copy measured with the same counters). Valid only for the kernel source whose
# sha256 starts with this prefix; reported as null for any other source.
GATE_UP_TRAFFIC = ("515145f85fe03e74", 9.89e9)
KERNEL_SOURCE = os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc", "bs_fp8_grouped.hip")


# The same for the 8192^3 launches (K = 8192) of other kernels: workload -> (source file, sha256
# prefix of that source, HBM bytes per launch).
SINGLE_TRAFFIC = {
    "nvfp4_8192": ("nv_fp4.hip", "0c838a70d41842ac", 0.590e9),
    "mx8192_e4m3_e4m3": ("mx_scaled.hip", "8de21e6fe08ece45", 1.064e9),
    "mx8192_e4m3_e2m1": ("mx_scaled.hip", "8de21e6fe08ece45", 0.842e9),
    "mx8192_e2m1_e2m1": ("mx_scaled.hip", "8de21e6fe08ece45", 0.572e9),
}
# ... and of other launches: one bsgemm_quantize_permute call (permute_rank + quantize kernels)
# of permute_moe32, one compact-layout small-M launch of decode_moe32, and one default launch
# (bsgemm_grouped_ws, large tiles) of the smaller blockwise workloads, partial tiles included.
OTHER_TRAFFIC = {
    "permute_moe32": ("permute.hip", "4db403de2891d156", 1.233e9),
    "decode_moe32": ("bs_fp8_small_m.hip", "edf5075f273bfb63", 0.907e9),
    "dense_4096": ("bs_fp8_grouped.hip", "515145f85fe03e74", 0.136e9),
    "moe8_n2048_k4096": ("bs_fp8_grouped.hip", "515145f85fe03e74", 0.325e9),
    "dense_256x2048x16384": ("bs_fp8_grouped.hip", "515145f85fe03e74", 0.119e9),
}


def _source_matches(path, prefix):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest().startswith(prefix)


def measured_traffic():
    return GATE_UP_TRAFFIC[1] if _source_matches(KERNEL_SOURCE, GATE_UP_TRAFFIC[0]) else None


def measured_traffic_single(workload, K):
    if workload not in SINGLE_TRAFFIC or K != 8192:
        return None
    src, prefix, nbytes = SINGLE_TRAFFIC[workload]
    path = os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc", src)
    return nbytes if _source_matches(path, prefix) else None


def measured_traffic_other(workload):
    if workload not in OTHER_TRAFFIC:
        return None
    src, prefix, nbytes = OTHER_TRAFFIC[workload]
    path = os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc", src)
    return nbytes if _source_matches(path, prefix) else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="moe32",
                    choices=["moe32", "mx8192_e4m3_e4m3", "mx8192_e4m3_e2m1", "mx8192_e2m1_e2m1",
                             "nvfp4_8192", "permute_moe32", "decode_moe32", "dense_4096",
                             "moe8_n2048_k4096", "dense_256x2048x16384"])
    ap.add_argument("--mx-k", type=int, default=8192, metavar="K",
                    help="K of the mx8192_* and nvfp4_8192 workloads (M = N = 8192; the pages' "
                         "K sweep runs 512 .. 8192)")
    ap.add_argument("--cold", action="store_true",
                    help="single-launch workloads: before each timed launch write 512 MiB of "
                         "scratch (untimed) so no operand is left in the caches; report the "
                         "median and minimum launch time")
    ap.add_argument("--no-split", action="store_true",
                    help="blockwise workloads: call bsgemm_grouped (whole work items only) instead of "
                         "bsgemm_grouped_ws (the last rounds of work items split along K)")
    ap.add_argument("--sched-small-m", action="store_true",
                    help="dense_4096 / moe8_n2048_k4096: request the one-M-tile-per-item schedule")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run --steps device-to-device copies of MIB "
                         "MiB each (a kernel of known traffic for scaling HBM counters) and exit")
    return ap.parse_args()


def cpu_baseline(problems, n_experts=8):
    """Time the oracle on a bounded sample of the step: every real row of the first ``n_experts``
    non-empty experts, for both GEMMs (gate_up and down). The oracle is the product by its
    definition (``blockwise_grouped_dequant``: decode and scale into fp64, then one BLAS product
    per expert). Returns the JSON object."""
    from threadpoolctl import threadpool_info

    from oracle import gemm as og
    from workloads.generate import padded_starts

    work, flops, rows = [], 0.0, 0
    for name in ("gate_up", "down"):
        p = problems[name]
        starts = padded_starts(p.counts)
        for e in [e for e in range(p.E) if p.counts[e] > 0][:n_experts]:
            r, s0 = int(p.counts[e]), int(starts[e])
            work.append((p.qa[s0:s0 + r].cpu().numpy(), p.a_scales[s0:s0 + r].cpu().numpy(),
                         p.qb[e].cpu().numpy(), p.b_scales[e].cpu().numpy()))
            flops += 2.0 * r * p.N * p.K
            rows += r
    t0 = time.perf_counter()
    for qa, sa, qb, sb in work:
        og.blockwise_grouped_dequant(qa, sa, qb, sb)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"gate_up (N={problems['gate_up'].N}, K={problems['gate_up'].K}) and down "
                  f"(N={problems['down'].N}, K={problems['down'].K}): every real row of the first "
                  f"{n_experts} non-empty experts of each ({rows} rows in all); fp64 oracle by its "
                  f"definition (decode and scale, then one BLAS product per expert); {dt:.1f} s",
    }


def cpu_baseline_mx(p, rows=8192):
    """Time the oracle on the first ``rows`` rows of A of the MX GEMM (all N, all K)."""
    from threadpoolctl import threadpool_info

    from oracle import gemm as og

    qa, sa = p.qa[:rows].cpu().numpy(), p.a_scales[:rows].cpu().numpy()
    qb, sb = p.qb.cpu().numpy(), p.b_scales.cpu().numpy()
    t0 = time.perf_counter()
    if p.scale_kind == "nv":
        og.nv_gemm(qa, sa, qb, sb)
    else:
        og.mx_gemm(qa, sa, qb, sb, p.fmt_a, p.fmt_b)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": 2.0 * rows * p.N * p.K / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows} rows of A of the {p.M}x{p.N}x{p.K} {KIND_NAME[p.scale_kind]} GEMM "
                  f"({p.fmt_a} x {p.fmt_b}), "
                  f"fp64 oracle (decode, then one product); {dt:.1f} s",
    }


KIND_NAME = {"mx": "MX", "nv": "nvfp4"}


def time_cold(torch, stream, launch, steps):
    """Per-launch times (ms) with a 512 MiB scratch write before each launch, outside the timed
    events, so the operands come from HBM rather than from the 256 MB last-level cache."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    times = []
    for _ in range(steps):
        scratch.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    del scratch
    return times


def bench_mx(args, torch, bsg, make_problem):
    """A step is one dense MX (or nvfp4) GEMM launch on a resident 8192 x 8192 x K problem."""
    nv = args.workload == "nvfp4_8192"
    if args.mx_k == 8192:
        p = make_problem(args.workload, device="cuda", seed=args.seed)
    elif nv:
        from workloads.generate import nv_problem
        if args.mx_k <= 0 or args.mx_k % 256:
            raise SystemExit("--mx-k must be a positive multiple of 256 for nvfp4")
        p = nv_problem(8192, 8192, args.mx_k, device="cuda", seed=args.seed)
    else:
        from workloads.generate import mx_problem
        if args.mx_k <= 0 or args.mx_k % 128:
            raise SystemExit("--mx-k must be a positive multiple of 128")
        fa, fb = args.workload.split("_")[1:]
        p = mx_problem(8192, 8192, args.mx_k, fa, fb, device="cuda", seed=args.seed)
    C = torch.empty(p.M, p.N, dtype=torch.float16, device="cuda")
    fmt = bsg.make_fmt(p.fmt_a, p.fmt_b, p.scale_kind, "f16")
    stream = torch.cuda.current_stream()

    def step():
        bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, None, None, C, p.M, p.N, p.K, fmt,
                           num_tiles=p.M // 128, num_experts=1, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # a step is one launch: the timed launches run back to back between two events on the launch
    # stream, so the per-launch time carries no event overhead
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    kernel_ms = a.elapsed_time(b) / args.steps
    cold = time_cold(torch, stream, step, args.steps) if args.cold else None
    flops = p.useful_flops
    if nv:
        # the products run on the f16 matrix instruction (the e4m3 scales are folded into f16
        # operands), so the f16 rate is the ceiling
        peak = PEAK_FP16_TFLOPS
    else:
        peak = PEAK_FP4_TFLOPS if (p.fmt_a, p.fmt_b) == ("e2m1", "e2m1") else PEAK_FP8_TFLOPS
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    scales = "e4m3 per 16" if nv else "e8m0 per 32"
    out = {
        "metric": f"TFLOP/s, {KIND_NAME[p.scale_kind]} GEMM {p.M}x{p.N}x{p.K} ({p.fmt_a} x {p.fmt_b}, "
                  f"{scales})",
        "value": round(value, 2), "unit": "TFLOP/s", "pct_of_peak": round(100.0 * value / peak, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"{p.fmt_a}x{p.fmt_b}", "data": "synthetic",
        "config": {"workload": f"{args.workload}: dense {KIND_NAME[p.scale_kind]} GEMM M=N=8192, "
                               f"K={p.K}, {scales} K, fp16 out", "K": p.K, "seed": args.seed},
        "kernels_ms": {"nvfp4" if nv else "mx": round(kernel_ms, 4)},
        **({"cold_ms": {"median": round(float(np.median(cold)), 4), "min": round(min(cold), 4),
                        "tflops_at_median": round(flops / (np.median(cold) * 1e-3) / 1e12, 1)}}
           if cold else {}),
        "roofline": {
            "kernel": "nv_fp4_kernel (f16 MFMA)" if nv else f"mx_kernel<{p.fmt_a}, {p.fmt_b}>",
            "bound": "mfma",
            "achieved": round(kernel_tflops, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(kernel_tflops / peak, 4),
            "traffic": measured_traffic_single(args.workload, p.K),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mx(p)
    print(json.dumps(out), flush=True)


def permute_bytes(tokens, top_k, K, M):
    """Algorithmic bytes of one quantise-and-permute call: bf16 token rows read once, every row
    of the grouped A (codes and scales, padding included) written once, picks read and their
    rows written once."""
    return tokens * K * 2 + M * K + M * (K // 128) * 4 + 2 * tokens * top_k * 4


def cpu_baseline_permute(x, ids, eo, M, sample=1024):
    """Time the oracle's quantise-and-permute on the first ``sample`` tokens."""
    from threadpoolctl import threadpool_info

    from oracle import permute as op

    xs = x[:sample].float().cpu().numpy()
    ids_s = ids[:sample]
    counts = op.route_counts(ids_s, len(eo) - 1)
    offs = np.concatenate([[0], np.cumsum(-(-counts // 128) * 128)])
    Ms = int(offs[-1])
    t0 = time.perf_counter()
    op.quantize_permute(xs, ids_s, offs, Ms)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    nbytes = permute_bytes(sample, ids.shape[1], xs.shape[1], Ms)
    return {
        "value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": f"first {sample} of {x.shape[0]} tokens (their {sample * ids.shape[1]} picks), "
                  f"oracle quantise + permute; {dt:.1f} s",
    }


def bench_permute(args, torch, bsg):
    """A step: route counts, tile map, and quantise + permute of the 32-expert MoE activations."""
    from workloads.generate import MOE32, activations, routing_counts, routing_topk

    T, k, E, K = MOE32["tokens"], MOE32["top_k"], MOE32["experts"], 7168
    counts_h = routing_counts(seed=args.seed, **MOE32)
    ids_h = routing_topk(counts_h, T, k, seed=args.seed)
    T_tiles = int(sum(-(-int(c) // 128) for c in counts_h))
    M = 128 * T_tiles
    x = activations(T, K, device="cuda", seed=args.seed)
    ids = torch.from_numpy(ids_h).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    eo = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    to = torch.empty(T_tiles + 1, dtype=torch.int32, device="cuda")
    ei = torch.empty(T_tiles, dtype=torch.int32, device="cuda")
    dest = torch.empty(T, k, dtype=torch.int32, device="cuda")
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(M, K // 128, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    launches = []

    def step(record):
        bsg.bsgemm_route_counts(ids, E, counts=counts, stream=stream)
        bsg.bsgemm_build_tiles(counts, T_tiles, padded=True, expert_offsets=eo, tile_offsets=to,
                               expert_ids=ei, stream=stream)
        a = torch.cuda.Event(enable_timing=True) if record else None
        if record:
            a.record(stream)
        bsg.bsgemm_quantize_permute(x, ids, eo, M, E, dest=dest, qa=qa, a_scales=sa, stream=stream)
        if record:
            b = torch.cuda.Event(enable_timing=True)
            b.record(stream)
            launches.append((a, b))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in launches]))
    nbytes = permute_bytes(T, k, K, M)
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "GB/s, quantise (e4m3, 1x128 fp32 scales) + permute of MoE token activations "
                  "into the grouped GEMM's A",
        "value": round(value, 1), "unit": "GB/s", "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16->e4m3", "data": "synthetic",
        "config": {"workload": f"permute_moe32: {T} tokens x top-{k} over {E} experts (Dirichlet(1.0), "
                               f"2 empty), bf16 rows of K={K} -> {M} padded rows of e4m3",
                   "tokens": T, "top_k": k, "experts": E, "K": K, "padded_rows": M, "seed": args.seed},
        "kernels_ms": {"quantize_permute": round(call_ms, 4)},
        "roofline": {
            "kernel": "permute_rank_kernel + quantize_kernel (one bsgemm_quantize_permute call)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic_other("permute_moe32"),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_permute(x, ids_h, eo.cpu().numpy(), M)
    print(json.dumps(out), flush=True)


def bench_decode(args, torch, bsg):
    """A step: the gate_up grouped GEMM of a 128-token decode batch, small-M schedule, with A in the
    compact layout (each expert's rows packed, so an expert's last M-tile is partial and the
    small-M kernel stops at its last 16-row fragment). The padded layout (every group a multiple
    of 128 rows) and the large-tile schedule are timed alongside for reference."""
    from workloads.generate import blockwise_problem, padded_starts, routing_counts

    route = dict(tokens=128, top_k=8, experts=32, alpha=1.0, n_empty=2)
    counts = routing_counts(seed=args.seed, **route)
    N, K, E = 4096, 7168, 32
    p = blockwise_problem(list(int(c) for c in counts), N, K, device="cuda", seed=args.seed)
    c = torch.tensor(counts, dtype=torch.int32, device="cuda")
    active = int(np.count_nonzero(counts))
    real = int(np.sum(counts))
    # the same rows packed: expert e's real rows of the padded A, one group after another
    starts = padded_starts(counts)
    keep = torch.as_tensor(np.concatenate([np.arange(starts[e], starts[e] + counts[e]) for e in range(E)]),
                           dtype=torch.int64, device="cuda")
    layouts = {}
    for name, qa, sa, M, padded in (("padded", p.qa, p.a_scales, p.M, True),
                                    ("compact", p.qa[keep].contiguous(), p.a_scales[keep].contiguous(), real, False)):
        T = int(sum(-(-int(x) // 128) for x in counts)) if not padded else p.M // 128
        _, to, ei = bsg.bsgemm_build_tiles(c, T, padded=padded)
        layouts[name] = (qa, sa, M, T, to, ei, torch.empty(M, N, dtype=torch.bfloat16, device="cuda"))
    stream = torch.cuda.current_stream()

    def nbytes_of(M):
        return (active * N * K + active * (N // 128) * (K // 128) * 4     # B and its scales
                + M * K + M * (K // 128) * 4 + real * N * 2)               # A, a_scales, C rows

    def time_fmt(layout, small, steps, warmup):
        qa, sa, M, T, to, ei, C = layouts[layout]
        fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16", small_m=small)
        call = lambda: bsg.bsgemm_grouped(qa, sa, p.qb, p.b_scales, ei, to, C, M, N, K,
                                          fmt, num_experts=E, stream=stream)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = []
        t0 = time.perf_counter()
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return wall, float(np.mean([a.elapsed_time(b) for a, b in ev]))

    times = {}
    for layout in ("padded", "compact"):
        for small in (False, True):
            times[(layout, small)] = time_fmt(layout, small, args.steps, args.warmup)
    ms_per_step, call_ms = times[("compact", True)]
    nbytes = nbytes_of(real)
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    T_c, T_p = layouts["compact"][3], layouts["padded"][3]
    out = {
        "metric": "GB/s, grouped blockwise-FP8 GEMM for a decode batch (B streamed once per expert)",
        "value": round(value, 1), "unit": "GB/s", "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": f"decode_moe32: 128 tokens x top-8 over 32 experts (Dirichlet(1.0), "
                               f"2 empty) = {real} rows, compact layout ({T_c} M-tiles; padded: {T_p}); "
                               f"gate_up N={N}, K={K}; bf16 out",
                   "tokens": 128, "top_k": 8, "experts": E, "rows": real, "m_tiles": T_c, "seed": args.seed},
        "kernels_ms": {f"{layout}_{'small_m' if small else 'large_tile'}": round(t[1], 4)
                       for (layout, small), t in times.items()},
        "useful_tflops": round(2.0 * real * N * K / (call_ms * 1e-3) / 1e12, 1),
        "roofline": {
            "kernel": "bw_fp8_small_m_kernel (gate_up, decode batch, compact layout)", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic_other("decode_moe32"),
        },
    }
    if not args.no_cpu_baseline:
        qa, sa, M, T, to, ei, _ = layouts["padded"]
        out["cpu_baseline"] = cpu_baseline_decode(p, counts, ei, to, nbytes_of(p.M))
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(p, counts, ei, to, nbytes, n_experts=4):
    """Time the oracle on the rows of the first ``n_experts`` non-empty experts; report GB/s of
    the same byte accounting scaled by the share of rows."""
    from threadpoolctl import threadpool_info

    from oracle import gemm as og

    eo, to_r, ei_r = og.tile_map(counts, p.M // 128)
    live = [e for e in range(len(counts)) if counts[e] > 0][:n_experts]
    rows = np.concatenate([np.arange(eo[e], eo[e] + counts[e]) for e in live])
    args = [t.cpu().numpy() for t in (p.qa, p.a_scales, p.qb, p.b_scales)]
    t0 = time.perf_counter()
    og.blockwise_grouped(*args, ei_r, to_r, rows=rows)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    share = len(live) / max(1, int(np.count_nonzero(counts)))
    return {
        "value": nbytes * share / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": f"rows of the first {len(live)} non-empty experts ({len(rows)} rows), fp64 oracle "
                  f"K block by K block; {dt:.1f} s",
    }


def bench_blockwise(args, torch, bsg, make_problem):
    """A step is the tile map (grouped workloads) plus one blockwise-FP8 GEMM launch, bf16 out."""
    from oracle import gemm as og
    from threadpoolctl import threadpool_info
    from workloads.generate import padded_starts

    p = make_problem(args.workload, device="cuda", seed=args.seed)
    dev = p.qa.device
    stream = torch.cuda.current_stream()
    C = torch.empty(p.M, p.N, dtype=torch.bfloat16, device=dev)
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16", small_m=args.sched_small_m)
    grouped = p.counts is not None
    T = p.M // 128
    if grouped:
        counts = torch.tensor(p.counts, dtype=torch.int32, device=dev)
        eo = torch.empty(p.E + 1, dtype=torch.int32, device=dev)
        to = torch.empty(T + 1, dtype=torch.int32, device=dev)
        ei = torch.empty(T, dtype=torch.int32, device=dev)

    ws = None if args.no_split else torch.empty(bsg.bsgemm_grouped_workspace_size(), dtype=torch.uint8,
                                                device=dev)

    def gemm():
        if ws is None:
            bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, ei if grouped else None,
                               to if grouped else None, C, p.M, p.N, p.K, fmt, num_tiles=T,
                               num_experts=p.E, stream=stream)
        else:
            bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, ei if grouped else None,
                                  to if grouped else None, C, p.M, p.N, p.K, fmt, ws, num_tiles=T,
                                  num_experts=p.E, stream=stream)

    def step():
        if grouped:
            bsg.bsgemm_build_tiles(counts, T, True, eo, to, ei, stream)
        gemm()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # The kernel's own duration: the same number of GEMM launches back to back between two
    # events on the launch stream (a pair of events around each launch of a kernel this short
    # adds about a tenth to it).
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        gemm()
    b.record(stream)
    torch.cuda.synchronize()
    kernel_ms = a.elapsed_time(b) / args.steps
    cold = time_cold(torch, stream, gemm, args.steps) if args.cold else None
    flops = p.useful_flops
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    desc = {"dense_4096": "one group 4096^3, every 64th row of A and B x100",
            "moe8_n2048_k4096": "8 experts, 4096 tokens x top-2, Dirichlet(0.5), N=2048, K=4096",
            "dense_256x2048x16384": "one group M=256, N=2048, K=16384 (8 work items, split along K "
                                    "by bsgemm_grouped_ws)"}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2), "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {desc[args.workload]}, blockwise e4m3 "
                               f"1x128/128x128 fp32 scales, bf16 out", "real_rows": p.real_rows,
                   "padded_rows": p.M, "N": p.N, "K": p.K, "experts": p.E, "seed": args.seed,
                   "entry_point": "bsgemm_grouped" if ws is None else "bsgemm_grouped_ws"},
        "kernels_ms": {"gemm": round(kernel_ms, 4)},
        **({"cold_ms": {"median": round(float(np.median(cold)), 4), "min": round(min(cold), 4),
                        "tflops_at_median": round(flops / (np.median(cold) * 1e-3) / 1e12, 1)}}
           if cold else {}),
        "roofline": {"kernel": "bw_fp8_small_m_kernel" if args.sched_small_m else "bw_fp8_grouped_kernel",
                     "bound": "mfma",
                     "achieved": round(kernel_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": (measured_traffic_other(args.workload)
                                 if ws is not None and not args.sched_small_m else None)},
    }
    if not args.no_cpu_baseline:
        # the oracle on about 10 s of work: dense, all 4096 rows; grouped, up to 512 real rows of
        # each expert
        if grouped:
            starts = padded_starts(p.counts)
            parts = [(e, int(starts[e]), min(512, int(p.counts[e]))) for e in range(p.E)
                     if p.counts[e] > 0]
        else:
            parts = [(0, 0, p.M)]
        work = [(p.qa[s0:s0 + r].cpu().numpy(), p.a_scales[s0:s0 + r].cpu().numpy(),
                 p.qb[e].cpu().numpy(), p.b_scales[e].cpu().numpy()) for e, s0, r in parts]
        t1 = time.perf_counter()
        for qa, sa, qb, sb in work:
            og.blockwise_grouped(qa, sa, qb, sb)
        dt = time.perf_counter() - t1
        rows = sum(r for _, _, r in parts)
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        out["cpu_baseline"] = {
            "value": 2.0 * rows * p.N * p.K / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} real rows x N={p.N} x K={p.K} of {args.workload}, fp64 oracle K "
                      f"block by K block; {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(under expert parallelism each GPU runs this GEMM on its own experts' share)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return

    import mx_grouped_gemm_amd as bsg
    from workloads.generate import make_problem

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bsg.load_library()

    if args.workload == "permute_moe32":
        bench_permute(args, torch, bsg)
        return
    if args.workload == "decode_moe32":
        bench_decode(args, torch, bsg)
        return
    if args.workload in ("dense_4096", "moe8_n2048_k4096", "dense_256x2048x16384"):
        bench_blockwise(args, torch, bsg, make_problem)
        return
    if args.workload != "moe32":
        bench_mx(args, torch, bsg, make_problem)
        return

    problems = {
        "gate_up": make_problem("moe32_gate_up_n4096_k7168", device="cuda", seed=args.seed),
        "down": make_problem("moe32_down_n7168_k2048", device="cuda", seed=args.seed),
    }
    gu, dn = problems["gate_up"], problems["down"]
    assert np.array_equal(gu.counts, dn.counts)
    counts = torch.tensor(gu.counts, dtype=torch.int32, device=dev)
    T = gu.M // 128
    expert_offsets = torch.empty(gu.E + 1, dtype=torch.int32, device=dev)
    tile_offsets = torch.empty(T + 1, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(T, dtype=torch.int32, device=dev)
    C_gu = torch.empty(gu.M, gu.N, dtype=torch.bfloat16, device=dev)
    C_dn = torch.empty(dn.M, dn.N, dtype=torch.bfloat16, device=dev)
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16")
    stream = torch.cuda.current_stream()
    ws = None if args.no_split else torch.empty(bsg.bsgemm_grouped_workspace_size(), dtype=torch.uint8,
                                                device=dev)

    def gemm(p, C):
        if ws is None:
            bsg.bsgemm_grouped(p.qa, p.a_scales, p.qb, p.b_scales, expert_ids, tile_offsets, C, p.M, p.N,
                               p.K, fmt, num_tiles=T, num_experts=p.E, stream=stream)
        else:
            bsg.bsgemm_grouped_ws(p.qa, p.a_scales, p.qb, p.b_scales, expert_ids, tile_offsets, C, p.M,
                                  p.N, p.K, fmt, ws, num_tiles=T, num_experts=p.E, stream=stream)

    names = ("tile_map", "gate_up", "down")
    ev = {n: [] for n in names}

    def step(record):
        def mark():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e
        a = mark() if record else None
        bsg.bsgemm_build_tiles(counts, T, True, expert_offsets, tile_offsets, expert_ids, stream)
        b = mark() if record else None
        gemm(gu, C_gu)
        c = mark() if record else None
        gemm(dn, C_dn)
        d = mark() if record else None
        if record:
            ev["tile_map"].append((a, b))
            ev["gate_up"].append((b, c))
            ev["down"].append((c, d))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    kernel_ms = {n: float(np.mean([s.elapsed_time(e) for s, e in ev[n]])) for n in names}
    useful = {n: p.useful_flops for n, p in problems.items()}
    total_flops = useful["gate_up"] + useful["down"]
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    gu_tflops = useful["gate_up"] / (kernel_ms["gate_up"] * 1e-3) / 1e12
    dn_tflops = useful["down"] / (kernel_ms["down"] * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {
            "workload": "moe32_16384tok_top8: tile map + gate_up (N=4096, K=7168) + down "
                        "(N=7168, K=2048), blockwise e4m3 1x128/128x128 fp32 scales, bf16 out",
            "experts": gu.E, "tokens": 16384, "top_k": 8, "real_rows": gu.real_rows,
            "padded_rows": gu.M, "m_tiles": T, "seed": args.seed,
            "entry_point": "bsgemm_grouped" if ws is None else "bsgemm_grouped_ws",
        },
        "kernels_ms": {n: round(v, 4) for n, v in kernel_ms.items()},
        "kernels_tflops": {"gate_up": round(gu_tflops, 1), "down": round(dn_tflops, 1)},
        "roofline": {
            "kernel": "bw_fp8_grouped_kernel (gate_up launch)",
            "bound": "mfma", "achieved": round(gu_tflops, 1), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gu_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": measured_traffic(),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(problems)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
