"""Thin ctypes binding of libtlc (include/tlc.h), with the same names.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Device buffers are torch tensors on the ROCm device (PyTorch supplies
device memory and streams); their ``data_ptr()`` is passed through.  A nonzero
status raises ``TLCError``.  If the shared library has not been built, loading
fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtlc.so")

OK = 0
ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_CAPACITY = -1, -2, -3, -4
ERR_HIP, ERR_TIMEOUT, ERR_BAD_PLAN = -5, -6, -7
MODE_AG, MODE_RS, MODE_MOE = 0, 1, 2
ORDER_NATURAL, ORDER_RANK_OFFSET = 0, 1
B_KN, B_NK = 0, 1
LAND_NONE, LAND_COPY_ENGINE, LAND_CU, LAND_MEMCPY, LAND_COLOCATED = 0, 1, 2, 3, 4
SCHED_DYNAMIC, SCHED_STATIC, SCHED_STREAMK = 0, 1, 2
MAX_WORLD = 32
EPOCH_MAX = 4096

EXPORTS = [
    "tlc_chunk_plan", "tlc_signals_alloc", "tlc_signals_free", "tlc_signals_set",
    "tlc_signals_clear_status", "tlc_read_status", "tlc_ag_gemm", "tlc_gemm_rs", "tlc_rs_reduce",
    "tlc_moe_plan_capacity", "tlc_moe_workspace_bytes", "tlc_moe_route", "tlc_ag_moe", "tlc_land",
    "tlc_status_string", "tlc_last_error", "tlc_version", "tlc_split_workspace_bytes", "tlc_streamk_workspace_bytes", "tlc_gemm_ar",
    "tlc_wall_clock_khz", "tlc_read_signals", "tlc_signals_rewind", "tlc_moe_route_static",
    "tlc_moe_static_workspace_bytes",
]


class TLCError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")
        self.status = status


class Tile(C.Structure):
    _fields_ = [("m0", C.c_int32), ("n0", C.c_int32), ("m_rows", C.c_int32), ("n_cols", C.c_int32),
                ("expert", C.c_int32), ("chunk_mask", C.c_uint32), ("key", C.c_int32),
                ("split", C.c_uint32)]


class PlanDesc(C.Structure):
    _fields_ = [("mode", C.c_int32), ("world", C.c_int32), ("rank", C.c_int32), ("M", C.c_int32),
                ("N", C.c_int32), ("rows_per_chunk", C.c_int32), ("bm", C.c_int32),
                ("bn", C.c_int32), ("order", C.c_int32), ("group_m", C.c_int32),
                ("split_k", C.c_int32), ("split_from", C.c_int32), ("sub_chunks", C.c_int32)]


class AGArgs(C.Structure):
    _fields_ = [("plan", C.c_void_p), ("n_tiles", C.c_int64), ("M", C.c_int32), ("N", C.c_int32),
                ("K", C.c_int32), ("world", C.c_int32), ("rank", C.c_int32),
                ("rows_per_chunk", C.c_int32), ("bm", C.c_int32), ("bn", C.c_int32),
                ("a", C.c_void_p), ("a_src", C.POINTER(C.c_void_p)), ("b", C.c_void_p),
                ("b_layout", C.c_int32), ("c", C.c_void_p), ("sig", C.c_void_p),
                ("epoch", C.c_uint32), ("land", C.c_int32), ("grid", C.c_int32),
                ("timeout_ns", C.c_int64), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_int64), ("schedule", C.c_int32), ("sub_chunks", C.c_int32),
                ("copy_wgs", C.c_int32), ("trace", C.c_void_p)]


class RSArgs(C.Structure):
    _fields_ = [("plan", C.c_void_p), ("n_tiles", C.c_int64), ("M", C.c_int32), ("N", C.c_int32),
                ("K", C.c_int32), ("world", C.c_int32), ("rank", C.c_int32),
                ("rows_per_chunk", C.c_int32), ("bm", C.c_int32), ("bn", C.c_int32),
                ("a", C.c_void_p), ("b", C.c_void_p), ("b_layout", C.c_int32),
                ("partials", C.c_void_p), ("remote_src", C.POINTER(C.c_void_p)),
                ("landing", C.POINTER(C.c_void_p)), ("out", C.c_void_p), ("sig", C.c_void_p),
                ("epoch", C.c_uint32), ("land", C.c_int32), ("grid", C.c_int32),
                ("timeout_ns", C.c_int64), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_int64), ("schedule", C.c_int32),
                ("send_dst", C.POINTER(C.c_void_p)), ("send_land", C.c_int32),
                ("send_stream", C.c_void_p)]


class SignalsBlock(C.Structure):
    """Host image of tlc_signals."""
    _fields_ = [("flags", C.c_uint32 * 32), ("land_count", C.c_uint32 * 32), ("status", C.c_int32 * 4),
                ("work_next", C.c_uint32), ("work_done", C.c_uint32), ("dest_done", C.c_uint32 * 32),
                ("dest_ready", C.c_uint32 * 32), ("reserved", C.c_uint32 * 122),
                ("epoch_table", C.c_uint32 * 4096)]


class ARArgs(C.Structure):
    _fields_ = [("rs", RSArgs), ("gathered_src", C.POINTER(C.c_void_p)), ("c", C.c_void_p),
                ("copy_wgs", C.c_int32)]


class MoERouteArgs(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("tokens_per_chunk", C.c_int32), ("world", C.c_int32),
                ("rank", C.c_int32), ("experts", C.c_int32), ("topk", C.c_int32),
                ("N", C.c_int32), ("bm", C.c_int32), ("bn", C.c_int32), ("order", C.c_int32),
                ("topk_idx", C.c_void_p), ("gates", C.c_void_p), ("counts", C.c_void_p),
                ("offsets", C.c_void_p), ("row_token", C.c_void_p), ("slot", C.c_void_p),
                ("plan", C.c_void_p), ("plan_cap", C.c_int64), ("n_tiles_dev", C.c_void_p),
                ("workspace", C.c_void_p), ("x", C.c_void_p), ("x_src", C.POINTER(C.c_void_p)),
                ("H", C.c_int32), ("sig", C.c_void_p), ("epoch", C.c_uint32)]


class MoEArgs(C.Structure):
    _fields_ = [("plan", C.c_void_p), ("n_tiles_dev", C.c_void_p), ("plan_cap", C.c_int64),
                ("row_token", C.c_void_p), ("tokens_per_chunk", C.c_int32), ("world", C.c_int32),
                ("rank", C.c_int32), ("experts", C.c_int32), ("topk", C.c_int32),
                ("H", C.c_int32), ("N", C.c_int32), ("bm", C.c_int32), ("bn", C.c_int32),
                ("x", C.c_void_p), ("x_src", C.POINTER(C.c_void_p)), ("w", C.c_void_p),
                ("w_layout", C.c_int32), ("y", C.c_void_p), ("sig", C.c_void_p),
                ("epoch", C.c_uint32), ("land", C.c_int32), ("grid", C.c_int32),
                ("timeout_ns", C.c_int64), ("schedule", C.c_int32), ("copy_wgs", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """Load libtlc.so (built by ``tile_level_communication_amd.build``); no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtlc.so is not built ({LIB_PATH}); run "
                               "`python -m tile_level_communication_amd.build` first")
        L = C.CDLL(LIB_PATH)
        st = C.c_int32
        vp = C.c_void_p
        L.tlc_chunk_plan.argtypes = [C.POINTER(PlanDesc), C.POINTER(Tile), C.c_int64,
                                     C.POINTER(C.c_int64), C.POINTER(C.c_int32)]
        L.tlc_chunk_plan.restype = st
        L.tlc_signals_alloc.argtypes = [C.POINTER(vp)]
        L.tlc_signals_alloc.restype = st
        L.tlc_signals_free.argtypes = [vp]
        L.tlc_signals_free.restype = st
        L.tlc_signals_set.argtypes = [vp, C.c_int32, C.c_uint32, vp]
        L.tlc_signals_set.restype = st
        L.tlc_signals_rewind.argtypes = [vp, vp]
        L.tlc_signals_rewind.restype = st
        L.tlc_signals_clear_status.argtypes = [vp, vp]
        L.tlc_signals_clear_status.restype = st
        L.tlc_read_status.argtypes = [vp, vp, C.POINTER(C.c_int32)]
        L.tlc_read_status.restype = st
        L.tlc_read_signals.argtypes = [vp, vp, C.POINTER(SignalsBlock)]
        L.tlc_read_signals.restype = st
        L.tlc_ag_gemm.argtypes = [C.POINTER(AGArgs), vp, C.POINTER(vp), C.c_int32]
        L.tlc_ag_gemm.restype = st
        L.tlc_gemm_rs.argtypes = [C.POINTER(RSArgs), vp, C.POINTER(vp), C.c_int32]
        L.tlc_gemm_rs.restype = st
        L.tlc_gemm_ar.argtypes = [C.POINTER(ARArgs), vp, C.POINTER(vp), C.c_int32]
        L.tlc_gemm_ar.restype = st
        L.tlc_rs_reduce.argtypes = [C.POINTER(RSArgs), vp]
        L.tlc_rs_reduce.restype = st
        L.tlc_moe_plan_capacity.argtypes = [C.c_int32] * 6
        L.tlc_moe_plan_capacity.restype = C.c_int64
        L.tlc_moe_workspace_bytes.argtypes = [C.c_int32] * 4
        L.tlc_moe_workspace_bytes.restype = C.c_int64
        L.tlc_moe_route.argtypes = [C.POINTER(MoERouteArgs), vp]
        L.tlc_moe_route.restype = st
        L.tlc_moe_route_static.argtypes = [C.POINTER(MoERouteArgs), vp]
        L.tlc_moe_route_static.restype = st
        L.tlc_moe_static_workspace_bytes.argtypes = []
        L.tlc_moe_static_workspace_bytes.restype = C.c_int64
        L.tlc_ag_moe.argtypes = [C.POINTER(MoEArgs), vp, C.POINTER(vp), C.c_int32]
        L.tlc_ag_moe.restype = st
        L.tlc_land.argtypes = [C.POINTER(vp), C.POINTER(vp), C.c_int64, C.c_int32, C.c_int32, vp,
                               C.c_uint32, C.c_int32, C.POINTER(vp), C.c_int32]
        L.tlc_land.restype = st
        L.tlc_status_string.argtypes = [st]
        L.tlc_status_string.restype = C.c_char_p
        L.tlc_last_error.argtypes = []
        L.tlc_last_error.restype = C.c_char_p
        L.tlc_wall_clock_khz.argtypes = []
        L.tlc_wall_clock_khz.restype = C.c_int64
        L.tlc_version.argtypes = []
        L.tlc_version.restype = C.c_int32
        L.tlc_split_workspace_bytes.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int32]
        L.tlc_split_workspace_bytes.restype = C.c_int64
        L.tlc_streamk_workspace_bytes.argtypes = [C.c_int32]
        L.tlc_streamk_workspace_bytes.restype = C.c_int64
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().tlc_status_string(s).decode()


def last_error() -> str:
    return lib().tlc_last_error().decode()


def wall_clock_khz() -> int:
    """Rate of the device clock the traces count in (kHz)."""
    return int(lib().tlc_wall_clock_khz())


def version() -> int:
    return lib().tlc_version()


def _check(s: int, where: str):
    if s != OK:
        raise TLCError(s, where, last_error())


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _streams(s):
    """A stream, a list of streams or None -> (host array of hipStream_t, count)."""
    if s is None:
        return None, 0
    items = list(s) if isinstance(s, (list, tuple)) else [s]
    arr = (C.c_void_p * len(items))()
    for i, x in enumerate(items):
        arr[i] = _stream(x) or None
    return arr, len(items)


def _ptr_array(items, world):
    arr = (C.c_void_p * world)()
    for i, t in enumerate(items):
        arr[i] = _ptr(t) if t is not None else None
    return arr


# ------------------------------------------------------------------ plan ----

def chunk_plan(mode, world, rank, M, N, rows_per_chunk, bm, bn, order=ORDER_RANK_OFFSET,
               group_m=1, split_k=0, split_from=0, sub_chunks=0):
    """tlc_chunk_plan.  Returns (units: int32 ndarray [n_units, 8], landing_order: list)."""
    d = PlanDesc(mode, world, rank, M, N, rows_per_chunk, bm, bn, order, group_m, split_k,
                 split_from, sub_chunks)
    n = C.c_int64(0)
    _check(lib().tlc_chunk_plan(C.byref(d), None, 0, C.byref(n), None), "tlc_chunk_plan")
    tiles = (Tile * max(n.value, 1))()
    n_land = (world - 1) * max(sub_chunks, 1)
    land = (C.c_int32 * max(n_land, 1))()
    _check(lib().tlc_chunk_plan(C.byref(d), tiles, n.value, C.byref(n), land), "tlc_chunk_plan")
    arr = np.ctypeslib.as_array(C.cast(tiles, C.POINTER(C.c_int32)), shape=(max(n.value, 1), 8))
    return arr[:n.value].copy(), [int(land[i]) for i in range(n_land)]


def split_tiles(plan) -> int:
    """Number of split tiles in a unit list (units with split index 0 and S >= 2)."""
    sp = np.asarray(plan)[:, 7].astype(np.int64) & 0xFFFFFFFF
    return int(np.count_nonzero(((sp & 0xFF) >= 2) & (((sp >> 8) & 0xFF) == 0)))


def split_workspace_bytes(n_split_tiles, split_k, bm, bn) -> int:
    return int(lib().tlc_split_workspace_bytes(n_split_tiles, split_k, bm, bn))


def streamk_workspace_bytes(grid=0) -> int:
    return int(lib().tlc_streamk_workspace_bytes(grid))


# --------------------------------------------------------------- signals ----

class Signals:
    """One tlc_signals block (fine-grained device memory) owned by Python."""

    def __init__(self):
        p = C.c_void_p()
        _check(lib().tlc_signals_alloc(C.byref(p)), "tlc_signals_alloc")
        self.ptr = p.value

    def set(self, world: int, value: int, stream=None):
        _check(lib().tlc_signals_set(self.ptr, world, value, _stream(stream)), "tlc_signals_set")

    def rewind(self, stream=None):
        _check(lib().tlc_signals_rewind(self.ptr, _stream(stream)), "tlc_signals_rewind")

    def clear_status(self, stream=None):
        _check(lib().tlc_signals_clear_status(self.ptr, _stream(stream)), "tlc_signals_clear_status")

    def read_status(self, stream=None):
        out = (C.c_int32 * 4)()
        _check(lib().tlc_read_status(self.ptr, _stream(stream), out), "tlc_read_status")
        return [int(v) for v in out]

    def read_block(self, stream=None) -> SignalsBlock:
        """tlc_read_signals: the whole block, copied to the host after `stream`."""
        out = SignalsBlock()
        _check(lib().tlc_read_signals(self.ptr, _stream(stream), C.byref(out)), "tlc_read_signals")
        return out

    def free(self):
        if self.ptr:
            _check(lib().tlc_signals_free(self.ptr), "tlc_signals_free")
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def signals_alloc() -> Signals:
    return Signals()


# ------------------------------------------------------------- AG-GEMM ------

def ag_gemm(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, a_src, b, b_layout, c,
            sig: Signals, epoch, land, compute_stream=None, copy_stream=None, grid=0, timeout_ns=0,
            trace=None, workspace=None, schedule=SCHED_DYNAMIC, sub_chunks=0, copy_wgs=0):
    """tlc_ag_gemm.  a_src: list of `world` device tensors (entry `rank` unused) or None.
    copy_stream: one stream or a list of streams for the landing.  workspace: a
    zero-filled device tensor for split plans (or None)."""
    src = _ptr_array(a_src, world) if a_src is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = AGArgs(_ptr(plan), n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, _ptr(a), src,
                  _ptr(b), b_layout, _ptr(c), sig.ptr, epoch, land, grid, timeout_ns,
                  _ptr(workspace), ws_bytes, schedule, sub_chunks, copy_wgs, _ptr(trace))
    cs, n = _streams(copy_stream)
    _check(lib().tlc_ag_gemm(C.byref(args), _stream(compute_stream), cs, n), "tlc_ag_gemm")


def _rs_args(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout, partials,
             remote_src, landing, out, sig, epoch, land, grid, timeout_ns, workspace=None,
             schedule=SCHED_DYNAMIC, send_dst=None, send_land=LAND_MEMCPY, send_stream=None):
    src = _ptr_array(remote_src, world) if remote_src is not None else None
    lnd = _ptr_array(landing, world) if landing is not None else None
    snd = _ptr_array(send_dst, world) if send_dst is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return RSArgs(_ptr(plan), n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, _ptr(a),
                  _ptr(b), b_layout, _ptr(partials), src, lnd, _ptr(out), sig.ptr, epoch, land,
                  grid, timeout_ns, _ptr(workspace), ws_bytes, schedule, snd, send_land,
                  _stream(send_stream))


def gemm_rs(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout, partials,
            remote_src, landing, out, sig: Signals, epoch, land, compute_stream=None,
            copy_stream=None, grid=0, timeout_ns=0, workspace=None, schedule=SCHED_DYNAMIC,
            send_dst=None, send_land=LAND_MEMCPY, send_stream=None):
    """tlc_gemm_rs.  remote_src, landing: lists of `world` device tensors (entry `rank` unused).
    send_dst: list of `world` device tensors (R x N f32, entry `rank` unused) receiving the
    partial slices P[c] once each is complete, on send_stream; None = no sends."""
    args = _rs_args(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout,
                    partials, remote_src, landing, out, sig, epoch, land, grid, timeout_ns,
                    workspace, schedule, send_dst, send_land, send_stream)
    cs, n = _streams(copy_stream)
    _check(lib().tlc_gemm_rs(C.byref(args), _stream(compute_stream), cs, n), "tlc_gemm_rs")


def gemm_ar(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout, partials,
            remote_src, landing, gathered_src, c, sig: Signals, epoch, land, compute_stream=None,
            copy_stream=None, grid=0, timeout_ns=0, workspace=None, schedule=SCHED_DYNAMIC,
            copy_wgs=0):
    """tlc_gemm_ar.  remote_src, landing, gathered_src: lists of `world` device tensors (entry
    `rank` unused); c: the M x N output."""
    rs = _rs_args(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout,
                  partials, remote_src, landing, None, sig, epoch, land, grid, timeout_ns,
                  workspace, schedule)
    g = _ptr_array(gathered_src, world) if gathered_src is not None else None
    args = ARArgs(rs, g, _ptr(c), copy_wgs)
    cs, n = _streams(copy_stream)
    _check(lib().tlc_gemm_ar(C.byref(args), _stream(compute_stream), cs, n), "tlc_gemm_ar")


def rs_reduce(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout, partials,
              remote_src, landing, out, sig: Signals, epoch, land=LAND_NONE, compute_stream=None,
              copy_stream=None, grid=0, timeout_ns=0):
    """tlc_rs_reduce: the reduce step only."""
    args = _rs_args(plan, n_tiles, M, N, K, world, rank, rows_per_chunk, bm, bn, a, b, b_layout,
                    partials, remote_src, landing, out, sig, epoch, land, grid, timeout_ns)
    _check(lib().tlc_rs_reduce(C.byref(args), _stream(compute_stream)), "tlc_rs_reduce")


# ---------------------------------------------------------------- AG-MoE ----

def moe_plan_capacity(T, topk, experts, N, bm, bn) -> int:
    return int(lib().tlc_moe_plan_capacity(T, topk, experts, N, bm, bn))


def moe_workspace_bytes(T, topk, experts, bm) -> int:
    return int(lib().tlc_moe_workspace_bytes(T, topk, experts, bm))


def moe_route(logits, tokens_per_chunk, world, rank, experts, topk, N, bm, bn, order, topk_idx,
              gates, counts, offsets, row_token, slot, plan, plan_cap, n_tiles_dev, workspace,
              stream=None, x=None, x_src=None, H=0, sig: "Signals" = None, epoch=0):
    """tlc_moe_route.  With x_src (list of `world` device tensors, entry `rank`
    unused) the top-k kernel also lands the peers' token chunks into x and
    raises their flags in sig to epoch (the co-located landing beside the
    routing)."""
    src = _ptr_array(x_src, world) if x_src is not None else None
    args = MoERouteArgs(_ptr(logits), tokens_per_chunk, world, rank, experts, topk, N, bm, bn,
                        order, _ptr(topk_idx), _ptr(gates), _ptr(counts), _ptr(offsets),
                        _ptr(row_token), _ptr(slot), _ptr(plan), plan_cap, _ptr(n_tiles_dev),
                        _ptr(workspace), _ptr(x) if x is not None else None, src, H,
                        sig.ptr if sig is not None else None, epoch)
    _check(lib().tlc_moe_route(C.byref(args), _stream(stream)), "tlc_moe_route")


def moe_route_static(logits, tokens_per_chunk, world, rank, experts, topk, N, bm, bn, order,
                     topk_idx, gates, counts, offsets, row_token, slot, plan, plan_cap,
                     n_tiles_dev, stream=None, x=None, x_src=None, H=0, sig: "Signals" = None,
                     epoch=0):
    """tlc_moe_route_static: tlc_moe_route with the library's static workspace
    (allocates nothing)."""
    src = _ptr_array(x_src, world) if x_src is not None else None
    args = MoERouteArgs(_ptr(logits), tokens_per_chunk, world, rank, experts, topk, N, bm, bn,
                        order, _ptr(topk_idx), _ptr(gates), _ptr(counts), _ptr(offsets),
                        _ptr(row_token), _ptr(slot), _ptr(plan), plan_cap, _ptr(n_tiles_dev),
                        None, _ptr(x) if x is not None else None, src, H,
                        sig.ptr if sig is not None else None, epoch)
    _check(lib().tlc_moe_route_static(C.byref(args), _stream(stream)), "tlc_moe_route_static")


def moe_static_workspace_bytes() -> int:
    return int(lib().tlc_moe_static_workspace_bytes())


def ag_moe(plan, n_tiles_dev, plan_cap, row_token, tokens_per_chunk, world, rank, experts, topk, H,
           N, bm, bn, x, x_src, w, w_layout, y, sig: Signals, epoch, land, compute_stream=None,
           copy_stream=None, grid=0, timeout_ns=0, schedule=SCHED_DYNAMIC, copy_wgs=0):
    src = _ptr_array(x_src, world) if x_src is not None else None
    args = MoEArgs(_ptr(plan), _ptr(n_tiles_dev), plan_cap, _ptr(row_token), tokens_per_chunk,
                   world, rank, experts, topk, H, N, bm, bn, _ptr(x), src, _ptr(w), w_layout,
                   _ptr(y), sig.ptr, epoch, land, grid, timeout_ns, schedule, copy_wgs)
    cs, n = _streams(copy_stream)
    _check(lib().tlc_ag_moe(C.byref(args), _stream(compute_stream), cs, n), "tlc_ag_moe")


def land(dst, src, bytes_per_chunk, world, rank, sig: Signals, epoch, land_kind, copy_stream=None):
    d = _ptr_array(dst, world)
    s = _ptr_array(src, world)
    cs, n = _streams(copy_stream)
    _check(lib().tlc_land(d, s, bytes_per_chunk, world, rank, sig.ptr, epoch, land_kind, cs, n),
           "tlc_land")
