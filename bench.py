#!/usr/bin/env python3
"""Benchmark: chunk-swizzled AllGather-GEMM on one MI355X.

Workload (default): the Qwen3-32B-like FFN-up AllGather-GEMM -- 8 chunks of
1024 x 5120 bf16 activations gathered into A (8192 x 5120), weight shard
B 5120 x 3200 bf16, C = A @ B in fp32.  One step = one pass of the whole path:
the 7 peer chunks land on a side stream (copy engine, one transfer per chunk,
then the chunk's flag), while the persistent tile-swizzled GEMM on the compute
stream starts with the local chunk and consumes the others as their flags
flip.  Inputs are seeded synthetic data already resident in HBM.

Reported (one JSON line): fused TFLOP/s (value), the GEMM kernel's roofline
(MFMA bf16 peak 2.5 PFLOP/s), compute-only and copy-only times and the overlap
efficiency eta = max(compute-only, copy-only) / fused, and the CPU oracle
timed on a bounded sample (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--land", default="copy_engine", choices=["copy_engine", "cu"])
    ap.add_argument("--layout", default="KN", choices=["KN", "NK"])
    ap.add_argument("--tile", type=int, default=256)
    ap.add_argument("--group-m", type=int, default=4)
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-only", action="store_true",
                    help="run the fused loop only (for rocprofv3), print nothing else")
    return ap.parse_args()


def timed(fn, steps, warmup, torch, streams):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(inp, budget_s):
    """The float64 oracle on a bounded sample of the workload: whole 1024-row
    chunks of C, as many as fit in about `budget_s` seconds."""
    import numpy as np
    from oracle import gemm as og
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    K, N = inp.b.shape
    R = inp.a_chunks[0].shape[0]
    flops = 0.0
    chunks = 0
    t0 = time.perf_counter()
    while True:
        c = chunks % len(inp.a_chunks)
        og.ag_gemm_rows(inp.a_chunks, inp.b, np.arange(c * R, (c + 1) * R))
        flops += 2.0 * R * N * K
        chunks += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{chunks} row chunks of {R}x{N} (K={K}) of C, float64, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the method (the other ranks are emulated on "
              "the same GPU); runs on more than one GPU are not supported.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import seeded_inputs as si
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import AGProblem

    wl = si.WORKLOADS[2]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = si.workload_inputs(2)
    layout = tlc.B_KN if args.layout == "KN" else tlc.B_NK
    land = tlc.LAND_COPY_ENGINE if args.land == "copy_engine" else tlc.LAND_CU
    prob = AGProblem(inp.a_chunks, inp.b, args.rank, args.tile, args.tile, layout,
                     group_m=args.group_m, device=dev)
    compute = torch.cuda.Stream(device=dev)
    copy = torch.cuda.Stream(device=dev)
    prob.streams.compute = compute
    prob.streams.copy = copy
    flops = prob.flops
    call = dict(plan=prob.plan, n_tiles=prob.n_tiles, M=prob.M, N=prob.N, K=prob.K, world=prob.world,
                rank=prob.rank, rows_per_chunk=prob.R, bm=args.tile, bn=args.tile, a=prob.a,
                b=prob.b, b_layout=layout, c=prob.c, sig=prob.sig)
    ev_pairs = []
    torch.cuda.synchronize()

    def fused():
        prob.epoch += 1
        copy.wait_stream(compute)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(compute)
        tlc.ag_gemm(**call, a_src=prob.a_src, epoch=prob.epoch, land=land, compute_stream=compute,
                    copy_stream=copy, grid=args.grid)
        e1.record(compute)
        compute.wait_stream(copy)
        ev_pairs.append((e0, e1))

    if args.profile_only:
        timed(fused, args.steps, args.warmup, torch, None)
        return

    # fused: landing + GEMM
    t_fused = timed(fused, args.steps, args.warmup, torch, None)
    durs = [a.elapsed_time(b) for a, b in ev_pairs[args.warmup:]]
    gemm_fused_ms = float(np.mean(durs))

    # compute-only: all chunks in place, flags preset once
    prob.place_all()
    prob.epoch += 1
    fixed_epoch = prob.epoch
    prob.sig.set(prob.world, fixed_epoch, compute)
    torch.cuda.synchronize()
    ev_pairs.clear()

    def compute_only():
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(compute)
        tlc.ag_gemm(**call, a_src=None, epoch=fixed_epoch, land=tlc.LAND_NONE,
                    compute_stream=compute, copy_stream=copy, grid=args.grid)
        e1.record(compute)
        ev_pairs.append((e0, e1))

    t_comp = timed(compute_only, args.steps, args.warmup, torch, None)
    gemm_comp_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_pairs[args.warmup:]]))

    # copy-only: the same landing sequence, no GEMM
    dst = [prob.a[c * prob.R:(c + 1) * prob.R] for c in range(prob.world)]

    def copy_only():
        prob.epoch += 1
        copy.wait_stream(compute)
        tlc.land(dst, prob.a_src, prob.R * prob.K * 2, prob.world, prob.rank, prob.sig, prob.epoch,
                 land, copy)
        compute.wait_stream(copy)

    t_copy = timed(copy_only, args.steps, args.warmup, torch, None)

    # device status of a final fused call (timeouts or plan errors would show here)
    torch.cuda.synchronize()
    fused()
    status = prob.sig.read_status(compute)

    value = flops / t_fused / 1e12
    achieved = flops / (gemm_fused_ms * 1e-3) / 1e12
    eta = max(t_comp, t_copy) / t_fused
    line = {
        "metric": "AG-GEMM TFLOP/s @1 GPU (fused landing + chunk-swizzled GEMM), % bf16 MFMA peak, overlap efficiency",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_fused * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, bf16)",
        "config": {"workload": wl.name, "M": prob.M, "N": prob.N, "K": prob.K, "world": prob.world,
                   "rank": prob.rank, "tile": [args.tile, args.tile, 64], "b_layout": args.layout,
                   "landing": args.land, "group_m": args.group_m, "n_tiles": prob.n_tiles,
                   "parallelism": "one GPU's share; peer ranks emulated by side-stream landings"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "gemm_kernel<256,256,KN,dense> (fused mode)"},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "compute_only_ms": round(t_comp * 1e3, 4),
        "compute_only_tflops": round(flops / t_comp / 1e12, 2),
        "gemm_kernel_ms": {"fused": round(gemm_fused_ms, 4), "compute_only": round(gemm_comp_ms, 4)},
        "copy_only_ms": round(t_copy * 1e3, 4),
        "copy_gbs": round(7 * prob.R * prob.K * 2 / t_copy / 1e9, 1),
        "overlap_efficiency": round(eta, 4),
        "device_status": status,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
