"""Device-side set-up of the three operations around the libtlc calls.

Each problem object owns its device buffers (torch tensors on the ROCm device),
its tile plan (built by ``tlc_chunk_plan`` or, for MoE, by ``tlc_moe_route`` on
the device) and a ``tlc_signals`` block, and exposes ``run()`` which enqueues
one call of the operation.  The emulated peers' data lives in separate source
buffers; every ``run()`` with landing enabled copies it in again and raises the
epoch, so each call waits for fresh arrivals.
"""
from __future__ import annotations

import numpy as np
import torch

from . import tlc


def to_bf16(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bf16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f32(x: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def weight_layout(b_kn: torch.Tensor, b_layout: int) -> torch.Tensor:
    """A K x N weight stored as K x N (KN) or as its N x K transpose (NK)."""
    return b_kn.contiguous() if b_layout == tlc.B_KN else b_kn.t().contiguous()


class Streams:
    """A compute stream (torch's current one) and `n_copy` side copy streams,
    all at the default priority.  Two copy streams let two copy engines land
    chunks at once."""

    def __init__(self, device, n_copy: int = 2):
        self.compute = torch.cuda.current_stream(device)
        self.copies = [torch.cuda.Stream(device=device) for _ in range(n_copy)]

    @property
    def copy(self):
        return self.copies

    def begin(self, land=None):
        """The landing may only overwrite buffers once earlier work is done.
        A step whose landing runs on the compute stream (co-located, or none)
        leaves the copy streams alone."""
        if land is not None and not uses_copy_streams(land):
            return
        for c in self.copies:
            c.wait_stream(self.compute)

    def end(self, land=None):
        if land is not None and not uses_copy_streams(land):
            return
        for c in self.copies:
            self.compute.wait_stream(c)


def uses_copy_streams(land) -> bool:
    """Whether a fused step with this landing enqueues work on the copy streams."""
    return land in (tlc.LAND_COPY_ENGINE, tlc.LAND_CU, tlc.LAND_MEMCPY)


# MoE landing mode of the Python layer: the chunks are landed by the routing's
# top-k kernel (tlc_moe_route with x_src), and tlc_ag_moe runs with
# TLC_LAND_NONE and the same epoch, waiting for their flags.
LAND_WITH_ROUTE = -1


def next_epoch(prob) -> int:
    """Advance the problem's epoch; copy-engine flags are raised from a table of
    TLC_EPOCH_MAX values, so past the end the flags are rewound to 0 and the
    epochs restart at 1."""
    prob.epoch += 1
    if prob.epoch > tlc.EPOCH_MAX:
        prob.streams.compute.synchronize()
        for c in prob.streams.copies:
            c.synchronize()
        prob.sig.rewind(prob.streams.compute)  # sub-chunk and ready flags included
        prob.epoch = 1
    return prob.epoch


def split_workspace(tiles, split_k, bm, bn, device):
    """Zero-filled workspace for the plan's split tiles (None if none is split)."""
    n = tlc.split_tiles(tiles)
    if n == 0:
        return None
    nbytes = tlc.split_workspace_bytes(n, split_k, bm, bn)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def streamk_workspace(device, grid=0):
    """Zeroed workspace of the stream-K tail for any grid (or `grid` workgroups)."""
    return torch.zeros(tlc.streamk_workspace_bytes(grid), dtype=torch.uint8, device=device)


def schedule_workspace(tiles, split_k, bm, bn, schedule, device):
    """The workspace a plan needs under `schedule`: the stream-K tail's, or the
    split tiles' (None if neither)."""
    if schedule == tlc.SCHED_STREAMK:
        return streamk_workspace(device)
    return split_workspace(tiles, split_k, bm, bn, device)


class AGProblem:
    def __init__(self, a_chunks, b_kn, rank, bm=256, bn=256, b_layout=tlc.B_KN,
                 order=tlc.ORDER_RANK_OFFSET, group_m=4, device="cuda", split_k=0, split_from=0,
                 schedule=tlc.SCHED_DYNAMIC, sub_chunks=0):
        self.device = torch.device(device)
        self.world = len(a_chunks)
        self.sub_chunks = sub_chunks
        self.rank = rank
        self.R, self.K = a_chunks[0].shape
        self.N = b_kn.shape[1]
        self.M = self.world * self.R
        self.bm, self.bn, self.b_layout = bm, bn, b_layout
        self.a_src = [to_bf16(a, self.device) for a in a_chunks]
        self.a = torch.empty((self.M, self.K), dtype=torch.bfloat16, device=self.device)
        self.a[rank * self.R:(rank + 1) * self.R].copy_(self.a_src[rank])
        self.b = weight_layout(to_bf16(b_kn, self.device), b_layout)
        self.c = torch.empty((self.M, self.N), dtype=torch.float32, device=self.device)
        tiles, self.landing_order = tlc.chunk_plan(tlc.MODE_AG, self.world, rank, self.M, self.N,
                                                   self.R, bm, bn, order, group_m, split_k,
                                                   split_from, sub_chunks)
        self.tiles = tiles
        self.plan = torch.from_numpy(tiles).to(self.device)
        self.n_tiles = int(tiles.shape[0])
        self.workspace = schedule_workspace(tiles, split_k, bm, bn, schedule, self.device)
        self.schedule = schedule
        self.sig = tlc.Signals()
        self.epoch = 0
        self.streams = Streams(self.device)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def place_all(self):
        """Copy every chunk into the gathered buffer (for compute-only runs)."""
        for c in range(self.world):
            self.a[c * self.R:(c + 1) * self.R].copy_(self.a_src[c])

    def poison_remote(self):
        """Fill the rows the landing will write with NaN (stale-read detector)."""
        for c in range(self.world):
            if c != self.rank:
                self.a[c * self.R:(c + 1) * self.R].fill_(float("nan"))

    def run(self, land=tlc.LAND_COPY_ENGINE, grid=0, timeout_ns=0, preset_flags=None, trace=None,
            copy_wgs=0):
        """Enqueue one AG-GEMM.  With land == LAND_NONE the flags are raised to the
        new epoch first (chunks must already be in place) unless preset_flags is
        False."""
        next_epoch(self)
        s = self.streams
        if land == tlc.LAND_NONE and preset_flags is not False:
            self.sig.set(self.world * max(self.sub_chunks, 1), self.epoch, s.compute)
        s.begin(land)
        tlc.ag_gemm(self.plan, self.n_tiles, self.M, self.N, self.K, self.world, self.rank, self.R,
                    self.bm, self.bn, self.a, self.a_src if land != tlc.LAND_NONE else None,
                    self.b, self.b_layout, self.c, self.sig, self.epoch, land, s.compute, s.copy,
                    grid, timeout_ns, trace, self.workspace, self.schedule, self.sub_chunks,
                    copy_wgs)
        s.end(land)

    def land_only(self, land=tlc.LAND_COPY_ENGINE):
        next_epoch(self)
        s = self.streams
        s.begin()
        dst = [self.a[c * self.R:(c + 1) * self.R] for c in range(self.world)]
        tlc.land(dst, self.a_src, self.R * self.K * 2, self.world, self.rank, self.sig, self.epoch,
                 land, s.copy)
        s.end()


class RSProblem:
    def __init__(self, a, b_kn, remote: dict, world, rank, bm=256, bn=256, b_layout=tlc.B_KN,
                 order=tlc.ORDER_RANK_OFFSET, group_m=4, device="cuda", split_k=0, split_from=0,
                 schedule=tlc.SCHED_DYNAMIC, sends=False):
        self.device = torch.device(device)
        self.world, self.rank = world, rank
        self.M, self.K = a.shape
        self.N = b_kn.shape[1]
        self.R = self.M // world
        self.bm, self.bn, self.b_layout = bm, bn, b_layout
        self.a = to_bf16(a, self.device)
        self.b = weight_layout(to_bf16(b_kn, self.device), b_layout)
        self.partials = torch.empty((self.M, self.N), dtype=torch.float32, device=self.device)
        self.out = torch.empty((self.R, self.N), dtype=torch.float32, device=self.device)
        self.remote_src = [None] * world
        self.landing = [None] * world
        for s in range(world):
            if s != rank:
                self.remote_src[s] = to_f32(remote[s], self.device)
                self.landing[s] = torch.empty((self.R, self.N), dtype=torch.float32, device=self.device)
        tiles, self.landing_order = tlc.chunk_plan(tlc.MODE_RS, world, rank, self.M, self.N, self.R,
                                                   bm, bn, order, group_m, split_k, split_from)
        self.tiles = tiles
        self.plan = torch.from_numpy(tiles).to(self.device)
        self.n_tiles = int(tiles.shape[0])
        self.workspace = schedule_workspace(tiles, split_k, bm, bn, schedule, self.device)
        self.schedule = schedule
        self.sig = tlc.Signals()
        self.epoch = 0
        self.streams = Streams(self.device)
        # the emulated peers' receive buffers for this rank's partial slices
        self.send_dst = None
        self.send_stream = None
        if sends:
            self.send_dst = [None if c == rank else
                             torch.empty((self.R, self.N), dtype=torch.float32, device=self.device)
                             for c in range(world)]
            self.send_stream = torch.cuda.Stream(device=self.device)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def reduce_bytes(self) -> int:
        return (self.world + 1) * self.R * self.N * 4

    def place_all(self):
        for s in range(self.world):
            if s != self.rank:
                self.landing[s].copy_(self.remote_src[s])

    def poison_remote(self):
        for s in range(self.world):
            if s != self.rank:
                self.landing[s].fill_(float("nan"))

    def _args(self):
        return (self.plan, self.n_tiles, self.M, self.N, self.K, self.world, self.rank, self.R,
                self.bm, self.bn, self.a, self.b, self.b_layout, self.partials)

    def run(self, land=tlc.LAND_COPY_ENGINE, grid=0, timeout_ns=0, send_land=None):
        """Enqueue one GEMM-RS; with send_land (and a problem built with sends)
        the partial slices are also sent to send_dst on send_stream."""
        next_epoch(self)
        s = self.streams
        if land == tlc.LAND_NONE:
            self.sig.set(self.world, self.epoch, s.compute)
        s.begin(land)
        send = send_land is not None and self.send_dst is not None
        if send:
            self.send_stream.wait_stream(s.compute)
        tlc.gemm_rs(*self._args(), self.remote_src if land != tlc.LAND_NONE else None, self.landing,
                    self.out, self.sig, self.epoch, land, s.compute, s.copy, grid, timeout_ns,
                    self.workspace, self.schedule, self.send_dst if send else None,
                    send_land if send else tlc.LAND_MEMCPY, self.send_stream if send else None)
        s.end(land)
        if send:
            s.compute.wait_stream(self.send_stream)

    def reduce_only(self, timeout_ns=0):
        next_epoch(self)
        s = self.streams
        self.sig.set(self.world, self.epoch, s.compute)
        tlc.rs_reduce(*self._args(), None, self.landing, self.out, self.sig, self.epoch,
                      tlc.LAND_NONE, s.compute, None, 0, timeout_ns)

    def land_only(self, land=tlc.LAND_COPY_ENGINE):
        next_epoch(self)
        s = self.streams
        s.begin()
        tlc.land(self.landing, self.remote_src, self.R * self.N * 4, self.world, self.rank, self.sig,
                 self.epoch, land, s.copy)
        s.end()


class ARProblem(RSProblem):
    """GEMM-AllReduce: the GEMM-RS problem plus the peers' reduced slices, which
    land into the other row chunks of the M x N output `c`."""

    def __init__(self, a, b_kn, remote: dict, gathered: dict, world, rank, bm=256, bn=256,
                 b_layout=tlc.B_KN, order=tlc.ORDER_RANK_OFFSET, group_m=4, device="cuda",
                 split_k=0, split_from=0, schedule=tlc.SCHED_DYNAMIC):
        super().__init__(a, b_kn, remote, world, rank, bm, bn, b_layout, order, group_m, device,
                         split_k, split_from, schedule)
        self.gathered_src = [None] * world
        for c in range(world):
            if c != rank:
                self.gathered_src[c] = to_f32(gathered[c], self.device)
        self.c = torch.empty((self.M, self.N), dtype=torch.float32, device=self.device)

    def place_all(self):
        super().place_all()
        for c in range(self.world):
            if c != self.rank:
                self.c[c * self.R:(c + 1) * self.R].copy_(self.gathered_src[c])

    def poison_remote(self):
        super().poison_remote()
        self.c.fill_(float("nan"))

    def run(self, land=tlc.LAND_COPY_ENGINE, grid=0, timeout_ns=0, copy_wgs=0):
        next_epoch(self)
        s = self.streams
        if land == tlc.LAND_NONE:
            self.sig.set(self.world, self.epoch, s.compute)
        s.begin(land)
        tlc.gemm_ar(*self._args(), self.remote_src if land != tlc.LAND_NONE else None, self.landing,
                    self.gathered_src if land != tlc.LAND_NONE else None, self.c, self.sig,
                    self.epoch, land, s.compute, s.copy, grid, timeout_ns, self.workspace,
                    self.schedule, copy_wgs)
        s.end(land)


class MoEProblem:
    def __init__(self, x_chunks, logits, w_ekn, rank, topk, bm=256, bn=256, b_layout=tlc.B_KN,
                 order=tlc.ORDER_RANK_OFFSET, device="cuda", schedule=tlc.SCHED_DYNAMIC):
        self.device = torch.device(device)
        self.schedule = schedule
        dev = self.device
        self.world = len(x_chunks)
        self.rank = rank
        self.Tc, self.H = x_chunks[0].shape
        self.T = self.world * self.Tc
        self.E, _, self.N = w_ekn.shape
        self.k = topk
        self.bm, self.bn, self.b_layout, self.order = bm, bn, b_layout, order
        self.x_src = [to_bf16(x, dev) for x in x_chunks]
        self.x = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=dev)
        self.x[rank * self.Tc:(rank + 1) * self.Tc].copy_(self.x_src[rank])
        w = to_bf16(w_ekn, dev)
        self.w = w.contiguous() if b_layout == tlc.B_KN else w.transpose(1, 2).contiguous()
        self.logits = to_f32(logits, dev)
        T, k, E = self.T, self.k, self.E
        i32 = dict(dtype=torch.int32, device=dev)
        self.topk_idx = torch.empty((T, k), **i32)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), **i32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.row_token = torch.empty((T * k,), **i32)
        self.slot = torch.empty((T, k), **i32)
        self.plan_cap = tlc.moe_plan_capacity(T, k, E, self.N, bm, bn)
        self.plan = torch.empty((self.plan_cap, 8), **i32)
        self.n_tiles_dev = torch.zeros((1,), **i32)
        ws = tlc.moe_workspace_bytes(T, k, E, bm)
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=dev)
        self.y = torch.empty((T * k, self.N), dtype=torch.float32, device=dev)
        self.sig = tlc.Signals()
        self.epoch = 0
        self.streams = Streams(dev)

    @property
    def flops(self) -> float:
        return 2.0 * self.T * self.k * self.N * self.H

    def place_all(self):
        for c in range(self.world):
            self.x[c * self.Tc:(c + 1) * self.Tc].copy_(self.x_src[c])

    def poison_remote(self):
        for c in range(self.world):
            if c != self.rank:
                self.x[c * self.Tc:(c + 1) * self.Tc].fill_(float("nan"))

    def route(self, land_chunks=False):
        """Routing on the compute stream; with land_chunks the top-k kernel also
        lands the peers' token chunks (co-located landing beside the routing)
        and raises their flags to the current epoch."""
        s = self.streams
        tlc.moe_route(self.logits, self.Tc, self.world, self.rank, self.E, self.k, self.N, self.bm,
                      self.bn, self.order, self.topk_idx, self.gates, self.counts, self.offsets,
                      self.row_token, self.slot, self.plan, self.plan_cap, self.n_tiles_dev,
                      self.workspace, s.compute, x=self.x if land_chunks else None,
                      x_src=self.x_src if land_chunks else None, H=self.H,
                      sig=self.sig if land_chunks else None, epoch=self.epoch)

    def run(self, land=tlc.LAND_COPY_ENGINE, grid=0, timeout_ns=0, do_route=True, copy_wgs=0):
        """One step: routing, then the grouped GEMM consuming the chunks as they
        land.  land: a TLC_LAND_* backend of tlc_ag_moe, or LAND_WITH_ROUTE (the
        routing's top-k kernel lands the chunks; the GEMM waits for their flags)."""
        next_epoch(self)
        s = self.streams
        with_route = land == LAND_WITH_ROUTE
        if land == tlc.LAND_NONE:
            self.sig.set(self.world, self.epoch, s.compute)
        s.begin(land)
        if do_route or with_route:
            self.route(land_chunks=with_route)
        gemm_land = tlc.LAND_NONE if with_route else land
        tlc.ag_moe(self.plan, self.n_tiles_dev, self.plan_cap, self.row_token, self.Tc, self.world,
                   self.rank, self.E, self.k, self.H, self.N, self.bm, self.bn, self.x,
                   self.x_src if gemm_land != tlc.LAND_NONE else None, self.w, self.b_layout, self.y,
                   self.sig, self.epoch, gemm_land, s.compute, s.copy, grid, timeout_ns,
                   schedule=self.schedule, copy_wgs=copy_wgs)
        s.end(land)

    def land_only(self, land=tlc.LAND_COPY_ENGINE):
        next_epoch(self)
        s = self.streams
        s.begin()
        dst = [self.x[c * self.Tc:(c + 1) * self.Tc] for c in range(self.world)]
        # the routing's landing is timed as the same load/store copy alone
        tlc.land(dst, self.x_src, self.Tc * self.H * 2, self.world, self.rank, self.sig, self.epoch,
                 tlc.LAND_COLOCATED if land == LAND_WITH_ROUTE else land, s.copy)
        s.end()
