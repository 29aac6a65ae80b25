#!/usr/bin/env python3
"""Benchmark of the chunk-swizzled overlap path on one MI355X.

Default line (--workload ag): the Qwen3-32B-like FFN-up AllGather-GEMM -- 8
chunks of 1024 x 5120 bf16 activations gathered into A (8192 x 5120), weight
shard B 5120 x 3200 bf16 (K x N), C = A @ B in fp32.  One step = one pass of the
whole path: the 7 peer chunks land on a side stream with hipMemcpyAsync (one
device-to-device transfer per chunk, then a 4-byte transfer raising the chunk's
flag), while the persistent tile-swizzled GEMM on the compute stream starts with
the local chunk and consumes the others as their flags flip.  The same step with
the transfers forced onto the SDMA engines, with the library's own copy kernel on
reserved compute units, and with the co-located backend (the GEMM's own
workgroups copy the chunks before computing) is reported beside it.

The same line carries the other half of the metric, GEMM-ReduceScatter, as the
sub-object "gemm_rs": the long-context FFN-down shape (A 131072 x 3200, B 3200 x
5120, 8 row chunks of 16384), scatter-order GEMM, the 7 remote partials landed
by hipMemcpyAsync and reduced into the local 16384 x 5120 slice, and the sends
of this rank's 7 partial slices to their owners gated on the GEMM's
per-destination ready flags (send tail in scatter and in natural order).

Other workloads (--workload rs | rs_long | ar | moe) print their own line.  Every
leg clears the status word (and the split workspace) first and reads it after:
a leg whose flag waits failed on the device reports no derived figure.

Inputs are seeded synthetic data resident in HBM when the timed region starts.
The CPU oracle is timed on a bounded sample of the same workload (cpu_baseline).
The dense lines also time the same product through the vendor library
(vendor_gemm: hipBLASLt behind torch, bf16 and fp32 outputs, both weight
layouts) as context for the GEMM's roofline fraction; --no-vendor skips it.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_SCLK_MHZ = 2400.0  # the clock the published MFMA peak is quoted at
PEAK_HBM_GBS = 8000.0
# Memory traffic per launch of each workload's dominant kernels (256 x 256 tiles,
# K x N weight), from rocprofv3 FETCH_SIZE and WRITE_SIZE passes (KiB per
# dispatch) recorded under profiles/, each scaled by what the same counter reads
# for work of known size: FETCH_SIZE x FETCH_SCALE, WRITE_SIZE x WRITE_SCALE.
# The one-workgroup GEMM of --workload fetch_calibration, which loads its 64 MiB
# of A and B once through the GEMM's own direct-to-LDS loads, reads FETCH_SIZE
# 32 830 KiB and WRITE_SIZE 256 KiB for its 256 KiB tile (the runtime's copy
# kernel reads half its loads too).  None where the kernel changed since the
# counters were taken.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
# fused steps queued ahead of the one whose units are traced (flag_spin)
TRACE_LEAD_STEPS = 4
TRAFFIC_KIB = {  # workload -> kernel -> (FETCH_SIZE, WRITE_SIZE) or None
    "ag": {"gemm": (222482.5, 102416.3)},
    "moe": {"gemm": (249696.4, 98304.0)},
    "rs": {"gemm": (50582.2, 65536.0), "reduce": (32788.8, 16385.8)},
    "ar": {"gemm": (50582.2, 65536.0), "reduce": (32788.8, 16385.8)},
    "rs_long": {"gemm": (3153934.1, 2621440.0), "reduce": (1310742.8, 327680.0)},
}


def traffic_bytes(workload, kernel):
    t = TRAFFIC_KIB[workload][kernel]
    if t is None:
        return None
    f, w = t
    return round((f * FETCH_SCALE + w * WRITE_SCALE) * 1024)


WORKLOAD_ID = {"ag": 2, "rs": 1, "rs_long": 3, "moe": 4, "ar": 1, "fetch_calibration": None}
LANDINGS = {"memcpy": 3, "copy_engine": 1, "cu": 2, "colocated": 4}  # tlc.LAND_*
ORDERS = {"natural": 0, "rank_offset": 1}  # tlc.ORDER_*
SCHEDULES = {"dynamic": 0, "static": 1, "streamk": 2}  # tlc.SCHED_*


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ag", choices=list(WORKLOAD_ID))
    ap.add_argument("--land", default="memcpy", choices=list(LANDINGS),
                    help="memcpy: hipMemcpyAsync device-to-device on the side stream (default); "
                         "copy_engine: the same forced onto the SDMA engines (NoCU); cu: our copy "
                         "kernel on reserved CUs; colocated: the GEMM's own workgroups copy first")
    ap.add_argument("--order", default="rank_offset", choices=list(ORDERS),
                    help="tile order: rank_offset (the chunk-following swizzle) or natural "
                         "(every rank walks the tiles from tile 0)")
    ap.add_argument("--legs", default="all", choices=["all", "headline"],
                    help="headline: only the named landing, its copy-only and the compute-only "
                         "step (for sweeps); all: every landing backend beside it")
    ap.add_argument("--no-rs", action="store_true",
                    help="ag: leave the GEMM-RS sub-object out of the line")
    ap.add_argument("--copy-wgs", type=int, default=0,
                    help="colocated: workgroups that copy (0 = the library's default)")
    ap.add_argument("--layout", default="KN", choices=["KN", "NK"])
    ap.add_argument("--tile", type=int, default=256)
    ap.add_argument("--group-m", type=int, default=8)
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--copy-streams", type=int, default=1)
    ap.add_argument("--split-k", type=int, default=None,
                    help="K ranges per split tile (default: 2 with the SDMA landing, none otherwise)")
    ap.add_argument("--split-from", type=int, default=None,
                    help="first key (chunk position) whose tiles are split (default 7)")
    ap.add_argument("--sub-chunks", type=int, default=None,
                    help="ag: land every peer chunk as S pieces with their own flags (default 1)")
    ap.add_argument("--schedule", default=None, choices=["dynamic", "static", "streamk"],
                    help="work distribution (default: static for ag, rs and ar; per landing for moe)")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip timing the same dense product through the vendor library")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="minimum busy time of each leg's warm-up (after the W warm-up steps)")
    return ap.parse_args(argv)


WARM_SECONDS = 0.5


def timed(fn, steps, warmup, torch):
    # W untimed warm-up steps, continued until the GPU has been busy with this
    # step for WARM_SECONDS: its clocks take that long to settle after an idle
    # gap, and the first measurement of a process otherwise runs slow
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < WARM_SECONDS:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def run_leg(prob, fn, steps, warmup, torch, stream):
    """One leg: status word (and split workspace) cleared first, the step timed,
    the status read after.  Returns (seconds per step, status[4])."""
    prob.sig.clear_status(stream)
    ws = getattr(prob, "workspace", None)
    if ws is not None:
        with torch.cuda.stream(stream):
            ws.zero_()
    torch.cuda.synchronize()
    t = timed(fn, steps, warmup, torch)
    return t, prob.sig.read_status(stream)


class KernelTimer:
    """HIP events around one launch on the stream the kernel runs on."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def __call__(self, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        self.pairs.append((e0, e1))

    def mean_ms(self, last):
        """Mean over the last `last` launches (the timed ones)."""
        import numpy as np
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs[-last:]]))


def flushed_ms(step, compute, steps, warmup, torch, dev):
    """Mean time of `step` (which orders its side streams after `compute` and
    joins them back) with the 256 MB MALL flushed before each one by a 512 MiB
    fill on `compute`: HIP events on `compute` after the fill and after the
    join, so the fill is not timed and the step's sources come from HBM."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    pairs = []
    for _ in range(warmup + steps):
        with torch.cuda.stream(compute):
            flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(compute)
        step()
        e1.record(compute)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    del flush
    return sum(a.elapsed_time(b) for a, b in pairs[warmup:]) / steps


def leg_summary(flops, t_fused, t_comp, t_copy, status):
    """Figures of one fused leg; a leg whose status word is nonzero skipped work,
    so none of its derived figures is given."""
    ok = status[0] == 0
    out = {"value": round(flops / t_fused / 1e12, 2) if ok else None,
           "ms_per_step": round(t_fused * 1e3, 4) if ok else None,
           "copy_only_ms": round(t_copy * 1e3, 4) if t_copy is not None else None,
           "overlap_efficiency": (round(max(t_comp, t_copy or 0.0) / t_fused, 4) if ok else None),
           "pct_peak": round(100 * flops / t_fused / 1e12 / PEAK_BF16_TFLOPS, 2) if ok else None,
           "device_status": status}
    if not ok:
        out["error"] = f"device status {status}: the leg's steps did not complete their work"
    return out


def other_landings(flops, t_comp, others, t_copy_others, extra_names=None):
    """The same step with the other landing backends, for the JSON line."""
    names = {v: k for k, v in LANDINGS.items()}
    names.update(extra_names or {})
    return {names[o]: leg_summary(flops, t_f, t_comp, t_copy_others.get(o), st)
            for o, (t_f, st) in others.items()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _oracle_sample(kind, inp, budget_s, rank, topk):
    import numpy as np
    from oracle import gemm as og
    flops = 0.0
    blocks = 0
    t0 = time.perf_counter()
    if kind == "ag":
        K, N = inp.b.shape
        R = inp.a_chunks[0].shape[0]
        while True:
            c = blocks % len(inp.a_chunks)
            og.ag_gemm_rows(inp.a_chunks, inp.b, np.arange(c * R, (c + 1) * R))
            flops += 2.0 * R * N * K
            blocks += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        what = f"{blocks} row chunks of {R}x{N} (K={K}) of C"
    elif kind == "moe":  # the routing once, then blocks of grouped-GEMM rows
        from oracle import moe as om
        r = om.route(inp.logits, topk, len(inp.x_chunks), rank, inp.x_chunks[0].shape[0])
        H, N = inp.w.shape[1], inp.w.shape[2]
        n_rows = int(r["offsets"][-1])
        rows = 1024
        while True:
            start = (blocks * rows) % n_rows
            idx = np.arange(start, min(start + rows, n_rows))
            om.grouped_gemm(inp.x_chunks, inp.w, r["offsets"], r["row_token"], idx)
            flops += 2.0 * len(idx) * N * H
            blocks += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        what = (f"routing of {inp.logits.shape[0]} tokens (top-{topk} of {inp.logits.shape[1]}), "
                f"then {blocks} blocks of up to {rows} grouped-GEMM rows (H={H}, N={N}); the "
                "routing's time is counted, its work is not")
    else:  # rs: rows of the local slice (partial GEMM + reduce)
        K, N = inp.b.shape
        W = len(inp.remote) + 1
        R = inp.a.shape[0] // W
        rows = 256
        while True:
            start = (blocks * rows) % R
            og.gemm_rs_rows(inp.a, inp.b, inp.remote, W, rank, np.arange(start, start + rows))
            flops += 2.0 * rows * N * K
            blocks += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        what = f"{blocks} blocks of {rows} rows of the reduced slice (K={K}, N={N})"
    dt = time.perf_counter() - t0
    return flops / dt / 1e12, what, dt


def cpu_baseline(kind, inp, budget_s, rank=0, topk=0):
    """The float64 oracle on a bounded sample of the workload (whole row blocks
    of the output, as many as fit in about `budget_s` seconds), with the BLAS
    thread pool as the host sets it and again with one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: no one-thread run
        threadpool_limits = None
        threads = os.cpu_count() or 1
    value, what, dt = _oracle_sample(kind, inp, budget_s, rank, topk)
    out = {"value": round(value, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{what}, float64, {dt:.1f} s",
           "nproc": os.cpu_count(), "cpu_model": _cpu_model()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            v1, what1, dt1 = _oracle_sample(kind, inp, budget_s / 2, rank, topk)
        out["one_thread"] = {"value": round(v1, 6), "cores": 1, "sample": f"{what1}, float64, {dt1:.1f} s"}
    return out


def vendor_gemm(torch, tlc, a, b, b_layout, gemm_ms):
    """The same product through the vendor library (hipBLASLt behind torch.matmul,
    and torch.mm with an fp32 output as this library writes), for a K x N and an
    N x K weight: context for the roofline fraction, never the measured path."""
    M, K = a.shape
    b_kn = (b if b_layout == tlc.B_KN else b.t()).contiguous()
    b_nk = b_kn.t().contiguous()
    flops = 2.0 * M * b_kn.shape[1] * K
    out = {"library": "hipBLASLt through torch.matmul (bf16 output) and torch.mm(out_dtype=float32)",
           "this_kernel_tflops": round(flops / gemm_ms / 1e9, 1)}
    variants = {"KN_bf16_out": lambda: torch.matmul(a, b_kn),
                "NK_bf16_out": lambda: torch.matmul(a, b_nk.t()),
                "KN_f32_out": lambda: torch.mm(a, b_kn, out_dtype=torch.float32),
                "NK_f32_out": lambda: torch.mm(a, b_nk.t(), out_dtype=torch.float32)}
    for name, fn in variants.items():
        try:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            out[name] = round(flops / (e0.elapsed_time(e1) / 20) / 1e9, 1)
        except Exception as e:  # an older torch without out_dtype
            out[name] = f"unavailable: {type(e).__name__}"
    del b_kn, b_nk
    torch.cuda.empty_cache()
    return out


def base_line(args, value, t_fused, extra):
    line = {
        "metric": "AG-GEMM / GEMM-RS TFLOP/s @1 GPU (fused landing + chunk-swizzled GEMM), "
                  "% bf16 MFMA peak, overlap efficiency",
        "value": round(value, 2) if value is not None else None,
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
    }
    line.update(extra)
    return line


def run_ag(args, torch, tlc, si, workloads):
    wl = si.WORKLOADS[2]
    dev = torch.device("cuda:0")
    inp = si.workload_inputs(2)
    layout = tlc.B_KN if args.layout == "KN" else tlc.B_NK
    land = LANDINGS[args.land]
    order = ORDERS[args.order]
    # fused plan: whole tiles; with the slow SDMA landing the last chunk's tiles
    # are cut in two along K, so that the tail after the last landing runs on
    # twice as many compute units
    split_k = (2 if land == tlc.LAND_COPY_ENGINE else 0) if args.split_k is None else args.split_k
    split_from = 7 if args.split_from is None else args.split_from
    # static slots: faster than the dynamic counter for the memcpy and the
    # co-located landings (one process each, two runs)
    args.schedule = args.schedule or "static"
    schedule = SCHEDULES[args.schedule]
    if schedule == tlc.SCHED_STREAMK:
        split_k = 0  # the tail's workspace replaces the split tiles'
    sub = 1 if args.sub_chunks is None else args.sub_chunks
    prob = workloads.AGProblem(inp.a_chunks, inp.b, args.rank, args.tile, args.tile, layout,
                               order=order, group_m=args.group_m, device=dev, split_k=split_k,
                               split_from=split_from * sub + (sub - 1), schedule=schedule,
                               sub_chunks=sub)
    compute = torch.cuda.Stream(device=dev)
    copies = [torch.cuda.Stream(device=dev) for _ in range(max(1, args.copy_streams))]
    prob.streams.compute = compute
    prob.streams.copies = copies
    flops = prob.flops
    call = dict(plan=prob.plan, n_tiles=prob.n_tiles, M=prob.M, N=prob.N, K=prob.K, world=prob.world,
                rank=prob.rank, rows_per_chunk=prob.R, bm=args.tile, bn=args.tile, a=prob.a,
                b=prob.b, b_layout=layout, c=prob.c, sig=prob.sig, workspace=prob.workspace,
                schedule=schedule, sub_chunks=sub)
    torch.cuda.synchronize()

    def fused_step(land_kind, timer=None):
        def step():
            workloads.next_epoch(prob)
            for c in copies:
                c.wait_stream(compute)
            run = lambda: tlc.ag_gemm(**call, a_src=prob.a_src, epoch=prob.epoch, land=land_kind,
                                      compute_stream=compute, copy_stream=copies, grid=args.grid,
                                      copy_wgs=args.copy_wgs)
            timer(run) if timer else run()
            for c in copies:
                compute.wait_stream(c)
        return step

    fused_t = KernelTimer(torch, compute)
    t_fused, status = run_leg(prob, fused_step(land, fused_t), args.steps, args.warmup, torch, compute)
    gemm_fused_ms = fused_t.mean_ms(args.steps)

    # per-unit trace stamps of a fused step: time the workgroups spent spinning
    # on chunk flags (the exposed part of the landing inside the GEMM).  The
    # traced step is the last of several queued back to back, as in the timed
    # loop: a step started from an idle GPU finds its copies already under way
    # and waits less.
    trace = torch.zeros((prob.n_tiles, 6), dtype=torch.int64, device=dev)
    prob.sig.clear_status(compute)
    torch.cuda.synchronize()
    for _ in range(TRACE_LEAD_STEPS):
        fused_step(land)()
    workloads.next_epoch(prob)
    for c in copies:
        c.wait_stream(compute)
    tlc.ag_gemm(**call, a_src=prob.a_src, epoch=prob.epoch, land=land, compute_stream=compute,
                copy_stream=copies, grid=args.grid, trace=trace, copy_wgs=args.copy_wgs)
    for c in copies:
        compute.wait_stream(c)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy()
    trace_status = prob.sig.read_status(compute)
    khz = max(tlc.wall_clock_khz(), 1)
    if trace_status[0] != 0 or (tr[:, 1:4] == 0).any():
        # units that stopped early carry no stamps: nothing to report
        spin = {"error": f"traced step ended with device status {trace_status}"}
    else:
        wait_us = (tr[:, 2] - tr[:, 1]) * 1e3 / khz
        span_us = float(tr[:, 3].max() - tr[:, 1].min()) * 1e3 / khz
        n_wg = len(set(tr[:, 0].tolist()))
        import numpy as np
        keys = prob.tiles[:, 6]
        spin = {"wait_us_total": round(float(wait_us.sum()), 1),
                "units_that_waited": int((wait_us > 1.0).sum()),
                "wait_fraction_of_workgroup_time": round(float(wait_us.sum()) / (n_wg * span_us), 4),
                "kernel_span_us": round(span_us, 1),
                # median wait of the units keyed by each landing position (0: the local chunk)
                "median_wait_us_by_position": [round(float(np.median(wait_us[keys == k])), 1)
                                               for k in range(int(keys.max()) + 1) if (keys == k).any()],
                "traced_step": f"the last of {TRACE_LEAD_STEPS + 1} steps queued back to back"}

    # the same step with the other landing backends (reported beside the headline)
    other_kinds = [o for o in LANDINGS.values() if o != land] if args.legs == "all" else []
    others = {o: run_leg(prob, fused_step(o), args.steps, args.warmup, torch, compute)
              for o in other_kinds}

    def copy_only_step(land_kind):
        # the landing sequence of the fused step alone (an AG call with no units)
        def step():
            workloads.next_epoch(prob)
            for c in copies:
                c.wait_stream(compute)
            tlc.ag_gemm(**dict(call, n_tiles=0), a_src=prob.a_src, epoch=prob.epoch, land=land_kind,
                        compute_stream=compute, copy_stream=copies, copy_wgs=args.copy_wgs)
            for c in copies:
                compute.wait_stream(c)
        return step

    t_copy, copy_status = run_leg(prob, copy_only_step(land), args.steps, args.warmup, torch, compute)
    copy_flushed_ms = (flushed_ms(copy_only_step(land), compute, args.steps, args.warmup, torch, dev)
                       if args.legs == "all" else None)
    t_copy_others = {o: run_leg(prob, copy_only_step(o), args.steps, args.warmup, torch, compute)[0]
                     for o in others}

    # compute-only: the GEMM alone, every chunk in place, no flag checks (land
    # NONE, epoch 0), whole tiles, static schedule -- its fastest configuration
    comp = workloads.AGProblem(inp.a_chunks, inp.b, args.rank, args.tile, args.tile, layout,
                               order=order, group_m=args.group_m, device=dev,
                               schedule=tlc.SCHED_STATIC)
    comp.place_all()
    comp.c = prob.c
    torch.cuda.synchronize()
    comp_t = KernelTimer(torch, compute)
    ccall = dict(call, plan=comp.plan, n_tiles=comp.n_tiles, a=comp.a, sig=comp.sig, workspace=None,
                 schedule=tlc.SCHED_STATIC, sub_chunks=0)

    def compute_only():
        comp_t(lambda: tlc.ag_gemm(**ccall, a_src=None, epoch=0, land=tlc.LAND_NONE,
                                   compute_stream=compute, copy_stream=None, grid=0))

    t_comp, comp_status = run_leg(comp, compute_only, args.steps, args.warmup, torch, compute)
    gemm_comp_ms = comp_t.mean_ms(args.steps)
    # five more compute-only launches with trace stamps, right after the
    # timed ones (clocks settled): the shader clock the workgroups ran at, from
    # their cycle counters against the constant-rate clock (the median of the
    # five launches: one launch now and then reads a momentary dip), and the
    # MFMA peak at that clock
    ctrace = torch.zeros((comp.n_tiles, 6), dtype=torch.int64, device=dev)
    sclk_samples = []
    for _ in range(5):
        tlc.ag_gemm(**ccall, a_src=None, epoch=0, land=tlc.LAND_NONE, compute_stream=compute,
                    copy_stream=None, grid=0, trace=ctrace)
        torch.cuda.synchronize()
        ct = ctrace.cpu().numpy()
        sclk_samples.append(float((ct[:, 5] - ct[:, 4]).sum())
                            / max(float((ct[:, 3] - ct[:, 2]).sum()), 1.0) * khz / 1e3)
    sclk_mhz = sorted(sclk_samples)[len(sclk_samples) // 2]
    achieved = flops / (gemm_comp_ms * 1e-3) / 1e12
    peak_at_sclk = PEAK_BF16_TFLOPS * sclk_mhz / PEAK_SCLK_MHZ
    head = leg_summary(flops, t_fused, t_comp, t_copy, status)
    extra = {
        "config": {"workload": wl.name, "M": prob.M, "N": prob.N, "K": prob.K, "world": prob.world,
                   "rank": prob.rank, "order": args.order, "tile": [args.tile, args.tile, 64],
                   "b_layout": args.layout, "landing": args.land, "copy_streams": len(copies),
                   "group_m": args.group_m, "n_units": prob.n_tiles, "split_k": split_k,
                   "split_from_chunk": split_from, "sub_chunks": sub, "schedule": args.schedule,
                   "parallelism": "one GPU's share; peer ranks emulated by side-stream landings"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (traffic_bytes("ag", "gemm") if args.tile == 256
                                 and args.layout == "KN" else None),
                     "traffic_unit": "bytes per launch past the L2 (calibrated FETCH_SIZE + WRITE_SIZE)",
                     "algorithmic_bytes": prob.M * prob.K * 2 + prob.K * prob.N * 2 + prob.M * prob.N * 4,
                     "kernel": "gemm_kernel_4w<KN,dense,no-wait>: compute-only launch, whole tiles, "
                               "static schedule, every chunk resident",
                     "sclk_mhz_measured": round(sclk_mhz, 1),
                     "sclk_mhz_samples": [round(x, 1) for x in sclk_samples],
                     "peak_at_measured_sclk": round(peak_at_sclk, 1),
                     "frac_at_measured_sclk": round(achieved / peak_at_sclk, 4),
                     "device_status": comp_status},
        "pct_peak": head["pct_peak"],
        "compute_only_ms": round(t_comp * 1e3, 4),
        "compute_only_tflops": round(flops / t_comp / 1e12, 2),
        "gemm_kernel_ms": {"fused": round(gemm_fused_ms, 4), "compute_only": round(gemm_comp_ms, 4)},
        "copy_only_ms": round(t_copy * 1e3, 4),
        "copy_only_ms_mall_flushed": round(copy_flushed_ms, 4) if copy_flushed_ms is not None else None,
        "copy_only_status": copy_status,
        "exposed_copy_ms": round((t_fused - t_comp) * 1e3, 4) if status[0] == 0 else None,
        "flag_spin": spin,
        "copy_gbs": round((prob.world - 1) * prob.R * prob.K * 2 / t_copy / 1e9, 1),
        "overlap_efficiency": head["overlap_efficiency"],
        "device_status": status,
        "other_landings": other_landings(flops, t_comp, others, t_copy_others),
    }
    if args.legs == "all":
        extra["full_grid"] = full_grid(args, torch, tlc, workloads, inp, layout, order, dev, compute,
                                       call, flops, khz, gemm_comp_ms, sclk_mhz)
    if not args.no_vendor:
        extra["vendor_gemm"] = vendor_gemm(torch, tlc, prob.a, prob.b, prob.b_layout, gemm_comp_ms)
    line = base_line(args, head["value"], t_fused, extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline("ag", inp, args.cpu_seconds)
    return line


def moe_hbm_view(gemm_s, prob, args):
    """The grouped GEMM's launch against the HBM peak: its algorithmic bytes
    (X read once, W once, Y written once) and its measured traffic past the L2
    (the counters' figures) per second of the same launch."""
    alg = prob.T * prob.H * 2 + prob.E * prob.H * prob.N * 2 + prob.T * prob.k * prob.N * 4
    traffic = traffic_bytes("moe", "gemm") if args.tile == 256 and args.layout == "KN" else None
    out = {"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "achieved": round(alg / gemm_s / 1e9, 1), "frac": round(alg / gemm_s / 1e9 / PEAK_HBM_GBS, 4),
           "algorithmic_bytes": alg}
    if traffic is not None:
        out["traffic_gbs"] = round(traffic / gemm_s / 1e9, 1)
        out["traffic_frac"] = round(traffic / gemm_s / 1e9 / PEAK_HBM_GBS, 4)
    return out


def full_grid(args, torch, tlc, workloads, inp, layout, order, dev, compute, call, flops, khz,
              base_ms, base_mhz):
    """The compute-only GEMM on every compute unit instead of the default grid
    (two even rounds of whole tiles): whole tiles on static slots (the second
    round part-filled), and the stream-K tail (one round of whole tiles, the
    rest split along K over every CU).  Each with the kernel's mean time (HIP
    events) and the shader clock its workgroups ran at (cycle counters of the
    whole-tile units in five traced launches, median), beside the default."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {"default": {"grid": "default", "gemm_ms": round(base_ms, 4),
                       "tflops": round(flops / base_ms / 1e9, 1), "sclk_mhz": round(base_mhz, 1)}}
    for name, sched in [("static", tlc.SCHED_STATIC), ("streamk", tlc.SCHED_STREAMK)]:
        comp = workloads.AGProblem(inp.a_chunks, inp.b, args.rank, args.tile, args.tile, layout,
                                   order=order, group_m=args.group_m, device=dev, schedule=sched)
        comp.place_all()
        torch.cuda.synchronize()
        timer = KernelTimer(torch, compute)
        kw = dict(call, plan=comp.plan, n_tiles=comp.n_tiles, a=comp.a, c=comp.c, sig=comp.sig,
                  workspace=comp.workspace, schedule=sched, sub_chunks=0)

        def launch(trace=None):
            tlc.ag_gemm(**kw, a_src=None, epoch=0, land=tlc.LAND_NONE, compute_stream=compute,
                        copy_stream=None, grid=cus, trace=trace)

        _, st = run_leg(comp, lambda: timer(launch), args.steps, args.warmup, torch, compute)
        ms = timer.mean_ms(args.steps)
        whole = comp.n_tiles // cus * cus if sched == tlc.SCHED_STREAMK else comp.n_tiles
        tr = torch.zeros((comp.n_tiles, 6), dtype=torch.int64, device=dev)
        mhz = []
        for _ in range(5):
            launch(tr)
            torch.cuda.synchronize()
            t = tr[:whole].cpu().numpy()
            mhz.append(float((t[:, 5] - t[:, 4]).sum()) / max(float((t[:, 3] - t[:, 2]).sum()), 1.0)
                       * khz / 1e3)
        ok = st[0] == 0
        out[name] = {"grid": cus, "gemm_ms": round(ms, 4) if ok else None,
                     "tflops": round(flops / ms / 1e9, 1) if ok else None,
                     "sclk_mhz": round(sorted(mhz)[2], 1), "device_status": st}
        del comp
    return out


def run_rs(args, torch, tlc, si, workloads, wid, ar=False, sub_object=False):
    """GEMM-RS; with ar=True GEMM-AllReduce on the same shape (the reduce-scatter
    plus the all-gather of the peers' reduced slices into the M x N output).
    sub_object: the figures for the AG line's "gemm_rs" entry."""
    wl = si.WORKLOADS[wid]
    dev = torch.device("cuda:0")
    if ar:
        inp = si.ar_inputs(wid, wl.world, args.rank, wl.rows_per_chunk, wl.n, wl.k, wl.a_std,
                           wl.b_std, wl.remote_std)
    else:
        inp = si.workload_inputs(wid, rank=args.rank)
    layout = tlc.B_KN if args.layout == "KN" else tlc.B_NK
    land = LANDINGS[args.land]
    order = ORDERS[args.order]
    split_k = 0 if (args.split_k is None or sub_object) else args.split_k
    split_from = 1 if args.split_from is None else args.split_from
    schedule_name = "static" if sub_object else (args.schedule or "static")
    schedule = SCHEDULES[schedule_name]
    if schedule == tlc.SCHED_STREAMK:
        split_k = 0
    if ar:
        prob = workloads.ARProblem(inp.a, inp.b, inp.remote, inp.gathered, wl.world, args.rank,
                                   args.tile, args.tile, layout, order=order, group_m=args.group_m,
                                   device=dev, split_k=split_k, split_from=split_from,
                                   schedule=schedule)
    else:
        prob = workloads.RSProblem(inp.a, inp.b, inp.remote, wl.world, args.rank, args.tile,
                                   args.tile, layout, order=order, group_m=args.group_m, device=dev,
                                   split_k=split_k, split_from=split_from, schedule=schedule,
                                   sends=True)
    ws = dict(workspace=prob.workspace, schedule=schedule)
    c_chunks = ([prob.c[c * prob.R:(c + 1) * prob.R] for c in range(prob.world)] if ar else None)
    compute = torch.cuda.Stream(device=dev)
    copies = [torch.cuda.Stream(device=dev) for _ in range(max(1, args.copy_streams))]
    prob.streams.compute = compute
    prob.streams.copies = copies
    grid = 0 if sub_object else args.grid

    def call(land_kind, remote, landing, gathered, epoch, stream_list, sends=None):
        if ar:
            tlc.gemm_ar(*prob._args(), remote, landing, gathered, prob.c, prob.sig, epoch,
                        land_kind, compute, stream_list, grid, copy_wgs=args.copy_wgs, **ws)
        else:
            tlc.gemm_rs(*prob._args(), remote, landing, prob.out, prob.sig, epoch, land_kind,
                        compute, stream_list, grid, **ws,
                        send_dst=prob.send_dst if sends is not None else None,
                        send_land=sends if sends is not None else tlc.LAND_MEMCPY,
                        send_stream=prob.send_stream if sends is not None else None)

    flops = prob.flops
    torch.cuda.synchronize()
    steps, warm = args.steps, args.warmup

    def fused_step(land_kind):
        def step():
            workloads.next_epoch(prob)
            for c in copies:
                c.wait_stream(compute)
            call(land_kind, prob.remote_src, prob.landing, getattr(prob, "gathered_src", None),
                 prob.epoch, copies)
            for c in copies:
                compute.wait_stream(c)
        return step

    def copy_only_step(land_kind):
        def step():
            workloads.next_epoch(prob)
            for c in copies:
                c.wait_stream(compute)
            # co-located: the reduce reads the partials in place, so only the
            # all-gather (GEMM-AllReduce) moves data
            if not (ar and land_kind == tlc.LAND_COLOCATED):
                tlc.land(prob.landing, prob.remote_src, prob.R * prob.N * 4, prob.world, prob.rank,
                         prob.sig, prob.epoch, land_kind, copies)
            if ar:
                tlc.land(c_chunks, prob.gathered_src, prob.R * prob.N * 4, prob.world, prob.rank,
                         prob.sig, prob.epoch, land_kind, copies)
            for c in copies:
                compute.wait_stream(c)
        return step

    t_fused, status = run_leg(prob, fused_step(land), steps, warm, torch, compute)
    other_kinds = ([o for o in LANDINGS.values() if o != land]
                   if (args.legs == "all" and not sub_object) else [])
    others = {o: run_leg(prob, fused_step(o), steps, warm, torch, compute) for o in other_kinds}
    t_copy, copy_status = run_leg(prob, copy_only_step(land), steps, warm, torch, compute)
    copy_flushed_ms = (flushed_ms(copy_only_step(land), compute, steps, warm, torch, dev)
                       if args.legs == "all" else None)
    t_copy_others = {o: run_leg(prob, copy_only_step(o), steps, warm, torch, compute)[0]
                     for o in others}

    # sends of this rank's partial slices to their owners, gated on the GEMM's
    # per-destination ready flags, in the problem's order and in natural order:
    # when the last send completes against when the GEMM alone ends
    sends = None
    if not ar and prob.world > 1:
        plans = {args.order: (prob.plan, prob.n_tiles)}
        other = "natural" if args.order == "rank_offset" else "rank_offset"
        t_o, _ = tlc.chunk_plan(tlc.MODE_RS, prob.world, prob.rank, prob.M, prob.N, prob.R,
                                args.tile, args.tile, ORDERS[other], args.group_m, split_k,
                                split_from)
        plans[other] = (torch.from_numpy(t_o).to(dev), int(t_o.shape[0]))
        sends = {}
        for name, (plan, n_tiles) in plans.items():
            prob.plan, prob.n_tiles = plan, n_tiles
            rec = []

            def send_step(rec=rec):
                workloads.next_epoch(prob)
                for c in copies:
                    c.wait_stream(compute)
                prob.send_stream.wait_stream(compute)
                e0, ec, es = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(compute)
                call(land, prob.remote_src, prob.landing, None, prob.epoch, copies, sends=tlc.LAND_MEMCPY)
                ec.record(compute)
                es.record(prob.send_stream)
                rec.append((e0, ec, es))
                for c in copies:
                    compute.wait_stream(c)
                compute.wait_stream(prob.send_stream)

            t_send, st_send = run_leg(prob, send_step, steps, warm, torch, compute)
            # the GEMM alone in this order (no landing, no sends), less the reduce
            prob.place_all()
            prob.sig.set(prob.world, tlc.EPOCH_MAX, compute)
            gt = KernelTimer(torch, compute)
            rt = KernelTimer(torch, compute)
            for _ in range(warm + steps):
                gt(lambda: call(tlc.LAND_NONE, None, prob.landing, None, tlc.EPOCH_MAX, None))
                rt(lambda: tlc.rs_reduce(*prob._args(), None, prob.landing, prob.out, prob.sig,
                                         tlc.EPOCH_MAX, tlc.LAND_NONE, compute))
            torch.cuda.synchronize()
            gemm_ms = gt.mean_ms(steps) - rt.mean_ms(steps)
            prob.sig.rewind(compute)
            prob.epoch = 0
            torch.cuda.synchronize()
            import numpy as np
            sends_done = float(np.median([a.elapsed_time(c) for a, _, c in rec[-steps:]]))
            comp_done = float(np.median([a.elapsed_time(b) for a, b, _ in rec[-steps:]]))
            ok = st_send[0] == 0
            sends[name] = {"step_ms": round(t_send * 1e3, 4) if ok else None,
                           "sends_done_ms": round(sends_done, 4) if ok else None,
                           "gemm_and_reduce_done_ms": round(comp_done, 4) if ok else None,
                           "gemm_alone_ms": round(gemm_ms, 4),
                           "send_tail_ms": round(sends_done - gemm_ms, 4) if ok else None,
                           "device_status": st_send}
        prob.plan, prob.n_tiles = plans[args.order]

    prob.place_all()
    prob.sig.set(prob.world, tlc.EPOCH_MAX, compute)
    torch.cuda.synchronize()
    comp_t = KernelTimer(torch, compute)

    def compute_only():
        comp_t(lambda: call(tlc.LAND_NONE, None, prob.landing, None, tlc.EPOCH_MAX, None))

    t_comp, comp_status = run_leg(prob, compute_only, steps, warm, torch, compute)
    prob.sig.set(prob.world, tlc.EPOCH_MAX, compute)
    red_t = KernelTimer(torch, compute)

    def reduce_only():
        red_t(lambda: tlc.rs_reduce(*prob._args(), None, prob.landing, prob.out, prob.sig,
                                    tlc.EPOCH_MAX, tlc.LAND_NONE, compute))

    timed(reduce_only, steps, warm, torch)
    red_ms = red_t.mean_ms(steps)
    # the same with the 256 MB MALL flushed before each launch (a 512 MiB
    # fill in between): the reduce's sources then come from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    red_f = KernelTimer(torch, compute)

    def reduce_flushed():
        with torch.cuda.stream(compute):
            flush.fill_(1)
        red_f(lambda: tlc.rs_reduce(*prob._args(), None, prob.landing, prob.out, prob.sig,
                                    tlc.EPOCH_MAX, tlc.LAND_NONE, compute))

    timed(reduce_flushed, steps, warm, torch)
    red_flushed_ms = red_f.mean_ms(steps)
    del flush
    reduce_status = prob.sig.read_status(compute)

    torch.cuda.synchronize()
    gemm_ms = comp_t.mean_ms(steps) - red_ms
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    red_gbs = prob.reduce_bytes / (red_ms * 1e-3) / 1e9
    head = leg_summary(flops, t_fused, t_comp, t_copy, status)
    name = wl.name.replace("rs_", "ar_", 1) if ar else wl.name
    extra = {
        "config": {"workload": name, "M": prob.M, "N": prob.N, "K": prob.K, "world": prob.world,
                   "rank": prob.rank, "order": args.order, "tile": [args.tile, args.tile, 64],
                   "b_layout": args.layout, "landing": args.land, "copy_streams": len(copies),
                   "n_units": prob.n_tiles, "split_k": split_k, "split_from": split_from,
                   "schedule": schedule_name,
                   "parallelism": "one GPU's share; peer ranks emulated by side-stream landings"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": (traffic_bytes("rs_long" if wid == 3 else ("ar" if ar else "rs"), "gemm")
                                 if args.tile == 256 and args.layout == "KN" else None),
                     "traffic_unit": "bytes per launch past the L2 (calibrated FETCH_SIZE + WRITE_SIZE)",
                     "algorithmic_bytes": prob.M * prob.K * 2 + prob.K * prob.N * 2 + prob.M * prob.N * 4,
                     "kernel": "gemm_kernel_4w (scatter order, no waits)",
                     "device_status": comp_status},
        "reduce_roofline": {"bound": "hbm", "achieved": round(red_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(red_gbs / PEAK_HBM_GBS, 4),
                            "traffic": traffic_bytes("rs_long" if wid == 3 else "rs", "reduce"),
                            "algorithmic_bytes": prob.reduce_bytes,
                            "kernel": "reduce_kernel", "ms": round(red_ms, 4),
                            "ms_mall_flushed": round(red_flushed_ms, 4),
                            "achieved_mall_flushed": round(prob.reduce_bytes / (red_flushed_ms * 1e-3) / 1e9, 1),
                            "device_status": reduce_status},
        "pct_peak": head["pct_peak"],
        "compute_only_ms": round(t_comp * 1e3, 4),
        "compute_only_tflops": round(flops / t_comp / 1e12, 2),
        "copy_only_ms": round(t_copy * 1e3, 4),
        "copy_only_ms_mall_flushed": round(copy_flushed_ms, 4) if copy_flushed_ms is not None else None,
        "copy_only_status": copy_status,
        "overlap_efficiency": head["overlap_efficiency"],
        "device_status": status,
    }
    if sends is not None:
        extra["sends"] = sends
    if not args.no_vendor:
        extra["vendor_gemm"] = vendor_gemm(torch, tlc, prob.a, prob.b, prob.b_layout, gemm_ms)
    if other_kinds:
        extra["other_landings"] = other_landings(flops, t_comp, others, t_copy_others)
    if sub_object:
        return {"metric": "GEMM-RS TFLOP/s (fused landing + scatter-order GEMM + reduce)",
                "value": head["value"], "unit": "TFLOP/s", "ms_per_step": head["ms_per_step"],
                "steps": steps, "warmup": warm, **extra}
    line = base_line(args, head["value"], t_fused, extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline("rs", inp, args.cpu_seconds, args.rank)
    return line


def run_moe(args, torch, tlc, si, workloads):
    wl = si.WORKLOADS[4]
    dev = torch.device("cuda:0")
    inp = si.workload_inputs(4)
    layout = tlc.B_KN if args.layout == "KN" else tlc.B_NK
    land = LANDINGS[args.land]
    order = ORDERS[args.order]
    # Schedule per landing unless one is given: with no landing or a co-located
    # one, static slots keep each XCD on a contiguous run of the expert-major
    # plan (its weights and token rows stay in that XCD's L2), 3 % faster than
    # the dynamic counter; beside a side-stream landing the dynamic counter
    # lets units whose chunks have landed go ahead (with the memcpy landing on
    # every CU the two are equal; with 32 CUs left to the CU landing, ~486
    # units no longer fit two static rounds of 224 and the counter balances
    # them, 1-2 % faster).
    forced = {"static": tlc.SCHED_STATIC, "dynamic": tlc.SCHED_DYNAMIC}.get(args.schedule)

    def schedule_for(land_kind):
        if forced is not None:
            return forced
        return tlc.SCHED_DYNAMIC if workloads.uses_copy_streams(land_kind) else tlc.SCHED_STATIC

    schedule = schedule_for(land)
    args.schedule = args.schedule or ("dynamic" if schedule == tlc.SCHED_DYNAMIC else "static")
    prob = workloads.MoEProblem(inp.x_chunks, inp.logits, inp.w, args.rank, wl.topk, args.tile,
                                args.tile, layout, order=order, device=dev, schedule=schedule)
    compute = torch.cuda.Stream(device=dev)
    copies = [torch.cuda.Stream(device=dev) for _ in range(max(1, args.copy_streams))]
    prob.streams.compute = compute
    prob.streams.copies = copies
    flops = prob.flops
    torch.cuda.synchronize()

    # fused step: routing on the compute stream while the peers' tokens land,
    # then the readiness-sorted grouped GEMM consuming chunks as they arrive
    def fused_step(land_kind):
        def step():
            prob.schedule = schedule_for(land_kind)
            prob.run(land_kind, grid=args.grid, copy_wgs=args.copy_wgs)
        return step

    t_fused, status = run_leg(prob, fused_step(land), args.steps, args.warmup, torch, compute)
    # besides the four backends of tlc_ag_moe: the chunks landed by the routing's
    # top-k kernel (copy-only timed as the same load/store copy alone)
    route_name = {workloads.LAND_WITH_ROUTE: "colocated_route"}
    other_kinds = ([o for o in [*LANDINGS.values(), workloads.LAND_WITH_ROUTE] if o != land]
                   if args.legs == "all" else [])
    others = {o: run_leg(prob, fused_step(o), args.steps, args.warmup, torch, compute)
              for o in other_kinds}
    t_copy, copy_status = run_leg(prob, lambda: prob.land_only(land), args.steps, args.warmup, torch,
                                  compute)
    t_copy_others = {o: run_leg(prob, lambda o=o: prob.land_only(o), args.steps, args.warmup, torch,
                                compute)[0]
                     for o in others}

    prob.place_all()
    torch.cuda.synchronize()
    route_t = KernelTimer(torch, compute)
    gemm_t = KernelTimer(torch, compute)

    def compute_only():
        route_t(prob.route)
        gemm_t(lambda: tlc.ag_moe(prob.plan, prob.n_tiles_dev, prob.plan_cap, prob.row_token, prob.Tc,
                                  prob.world, prob.rank, prob.E, prob.k, prob.H, prob.N, prob.bm,
                                  prob.bn, prob.x, None, prob.w, prob.b_layout, prob.y, prob.sig, 0,
                                  tlc.LAND_NONE, compute, None, args.grid,
                                  schedule=schedule_for(tlc.LAND_NONE)))

    t_comp, comp_status = run_leg(prob, compute_only, args.steps, args.warmup, torch, compute)
    torch.cuda.synchronize()
    gemm_ms = gemm_t.mean_ms(args.steps)
    route_ms = route_t.mean_ms(args.steps)
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    head = leg_summary(flops, t_fused, t_comp, t_copy, status)
    extra = {
        "config": {"workload": wl.name, "tokens": prob.T, "experts": prob.E, "topk": prob.k,
                   "H": prob.H, "N": prob.N, "world": prob.world, "rank": prob.rank,
                   "order": args.order, "landing": args.land, "tile": [args.tile, args.tile, 64],
                   "n_tiles": int(prob.n_tiles_dev.item()), "schedule": args.schedule,
                   "parallelism": "one GPU's share; peer ranks emulated by side-stream landings"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (traffic_bytes("moe", "gemm") if args.tile == 256
                                 and args.layout == "KN" else None),
                     "traffic_unit": "bytes per launch past the L2 (calibrated FETCH_SIZE + WRITE_SIZE)",
                     "algorithmic_bytes": prob.T * prob.H * 2 + prob.E * prob.H * prob.N * 2
                     + prob.T * prob.k * prob.N * 4,
                     "kernel": "gemm_kernel_4w<KN,moe,no-wait,whole-tile loop>: grouped GEMM, every chunk resident",
                     "device_status": comp_status},
        # the grouped GEMM sits at the ridge point (2H flops per output element
        # against the bytes of X, W and Y: 323 flop/B, the peaks' ratio 312), so
        # the memory side of the same launch beside the MFMA fraction
        "roofline_hbm": moe_hbm_view(flops / (achieved * 1e12), prob, args),
        "route_ms": round(route_ms, 4),
        "pct_peak": head["pct_peak"],
        "compute_only_ms": round(t_comp * 1e3, 4),
        "compute_only_tflops": round(flops / t_comp / 1e12, 2),
        "copy_only_ms": round(t_copy * 1e3, 4),
        "copy_only_status": copy_status,
        "overlap_efficiency": head["overlap_efficiency"],
        "device_status": status,
        "other_landings": other_landings(flops, t_comp, others, t_copy_others, route_name),
    }
    line = base_line(args, head["value"], t_fused, extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline("moe", inp, args.cpu_seconds, args.rank, wl.topk)
    return line


def run_fetch_calibration(args, torch, tlc, si, workloads):
    """Known traffic for the memory counters: one workgroup computes one 256 x
    256 tile over K = 65536, so every byte of A (256 x K) and B (K x 256) is
    loaded exactly once, by the GEMM's own direct-to-LDS loads, and C (256 x
    256 fp32) is written once.  rocprofv3's FETCH_SIZE and WRITE_SIZE for these
    launches against the bytes below give the counters' scale for this kernel."""
    import numpy as np
    dev = torch.device("cuda:0")
    K, R, N = 65536, 256, 256
    inp = si.ag_inputs(900, 1, R, N, K)
    prob = workloads.AGProblem(inp.a_chunks, inp.b, 0, 256, 256, tlc.B_KN, device=dev,
                               schedule=tlc.SCHED_STATIC)
    prob.place_all()
    s = prob.streams.compute
    kt = KernelTimer(torch, s)
    fn = lambda: kt(lambda: tlc.ag_gemm(prob.plan, prob.n_tiles, prob.M, prob.N, prob.K, 1, 0, R,
                                        256, 256, prob.a, None, prob.b, tlc.B_KN, prob.c, prob.sig,
                                        0, tlc.LAND_NONE, s, None, 1, schedule=tlc.SCHED_STATIC))
    t, st = run_leg(prob, fn, args.steps, args.warmup, torch, s)
    return {"metric": "memory-counter calibration: bytes a one-workgroup GEMM moves",
            "workload": f"AG-GEMM M={R} N={N} K={K}, grid 1, one tile",
            "bytes_loaded": 2 * R * K + 2 * K * N, "bytes_stored": 4 * R * N,
            "launches": args.warmup + args.steps, "kernel_ms": round(kt.mean_ms(args.steps), 4),
            "device_status": st}


def main():
    global WARM_SECONDS
    args = parse()
    WARM_SECONDS = args.warm_seconds
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the method (the other ranks are emulated on "
              "the same GPU); runs on more than one GPU are not supported.", file=sys.stderr)
        sys.exit(2)
    import torch

    import seeded_inputs as si
    from tile_level_communication_amd import tlc, workloads

    torch.cuda.set_device(0)
    if args.workload == "fetch_calibration":
        print(json.dumps(run_fetch_calibration(args, torch, tlc, si, workloads)), flush=True)
        return
    if args.workload == "ag":
        line = run_ag(args, torch, tlc, si, workloads)
        if not args.no_rs:
            # the GEMM-RS half of the metric: the long-context FFN-down shape
            # with the landing and order of the headline
            line["gemm_rs"] = run_rs(args, torch, tlc, si, workloads, WORKLOAD_ID["rs_long"],
                                     sub_object=True)
    elif args.workload == "moe":
        line = run_moe(args, torch, tlc, si, workloads)
    else:
        line = run_rs(args, torch, tlc, si, workloads, WORKLOAD_ID[args.workload],
                      ar=args.workload == "ar")
    void_on_device_error(line, tlc)
    print(json.dumps(line), flush=True)


def void_on_device_error(line, tlc):
    """A flag wait that timed out on the device (status[0] != 0) means units were
    skipped: the headline steps measured incomplete work, so no figure derived
    from them is given."""
    st = line.get("device_status") or [0]
    if st[0] != 0:
        for k in ("value", "pct_peak", "overlap_efficiency", "exposed_copy_ms"):
            if k in line:
                line[k] = None
        line["error"] = (f"device status {st}: {tlc.status_string(st[0])}; "
                         "the timed fused steps did not complete their work")


if __name__ == "__main__":
    main()
