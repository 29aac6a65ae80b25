"""The C-ABI library loads and exports every function include/tlc.h declares
(no compute calls: no GPU is needed), and host-side argument validation
returns synchronous error codes."""
import ctypes as C
import os
import re

import pytest

from tile_level_communication_amd import tlc

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tlc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tlc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    assert set(names) == set(tlc.EXPORTS), names


def test_library_exports_every_declared_symbol():
    L = tlc.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert C.cast(getattr(L, name), C.c_void_p).value


def test_version_and_strings():
    assert tlc.version() == 132
    assert tlc.status_string(tlc.ERR_TIMEOUT).startswith("timeout")
    assert tlc.status_string(0) == "ok"


def test_struct_sizes_match_header():
    assert C.sizeof(tlc.Tile) == 32
    assert C.sizeof(tlc.PlanDesc) == 52


def _ag_args(**over):
    base = dict(plan=None, n_tiles=0, M=256, N=256, K=512, world=2, rank=0, rows_per_chunk=128,
                bm=128, bn=128, a=None, a_src=None, b=None, b_layout=tlc.B_KN, c=None, sig=None,
                epoch=1, land=tlc.LAND_NONE, grid=0, timeout_ns=0)
    base.update(over)
    return tlc.AGArgs(**base)


@pytest.mark.parametrize("over,want", [
    (dict(world=0), tlc.ERR_INVALID_ARG),
    (dict(rank=2), tlc.ERR_INVALID_ARG),
    (dict(M=255), tlc.ERR_INVALID_ARG),
    (dict(K=500), tlc.ERR_UNSUPPORTED),
    (dict(N=250, M=256), tlc.ERR_UNSUPPORTED),
    (dict(bm=64, bn=64), tlc.ERR_UNSUPPORTED),
    (dict(b_layout=7), tlc.ERR_INVALID_ARG),
    (dict(), tlc.ERR_INVALID_ARG),                       # NULL operands
    (dict(a=16, b=32, c=48, sig=64, n_tiles=4), tlc.ERR_INVALID_ARG),   # NULL plan
    (dict(a=8, b=32, c=48, sig=64), tlc.ERR_MISALIGNED),
    (dict(a=16, b=32, c=48, sig=64, land=9), tlc.ERR_INVALID_ARG),
    (dict(a=16, b=32, c=48, sig=64, land=tlc.LAND_CU), tlc.ERR_INVALID_ARG),  # no a_src
    (dict(a=16, b=32, c=48, sig=64, schedule=5), tlc.ERR_INVALID_ARG),
    (dict(a=16, b=32, c=48, sig=64, workspace_bytes=1024), tlc.ERR_INVALID_ARG),  # NULL workspace
    (dict(a=16, b=32, c=48, sig=64, workspace=4112, workspace_bytes=1024), tlc.ERR_MISALIGNED),
])
def test_ag_gemm_argument_errors(over, want):
    args = _ag_args(**over)
    s = tlc.lib().tlc_ag_gemm(C.byref(args), None, None, 0)
    assert s == want, tlc.last_error()
    assert tlc.last_error()


def test_colocated_landing_argument_errors():
    # the co-located landing raises flags from the kernel: epoch 0 would mean
    # "already landed" and is refused; no copy streams are needed
    src = (C.c_void_p * 2)(4096, 8192)
    args = _ag_args(a=16, b=32, c=48, sig=64, land=tlc.LAND_COLOCATED, epoch=0,
                    a_src=C.cast(src, C.POINTER(C.c_void_p)))
    assert tlc.lib().tlc_ag_gemm(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG
    assert "epoch" in tlc.last_error()
    d = (C.c_void_p * 2)(4096, 8192)
    s = tlc.lib().tlc_land(d, src, 1024, 2, 0, C.c_void_p(64), 0, tlc.LAND_COLOCATED, None, 0)
    assert s == tlc.ERR_INVALID_ARG and "epoch" in tlc.last_error()


def test_empty_sizes_are_refused():
    """Zero rows, columns, K or tokens: refused on the host with INVALID_ARG
    before anything is enqueued (no GPU is touched)."""
    for over in (dict(M=0, rows_per_chunk=0), dict(N=0), dict(K=0), dict(rows_per_chunk=0)):
        args = _ag_args(a=16, b=32, c=48, sig=64, **over)
        assert tlc.lib().tlc_ag_gemm(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG, over
        assert tlc.last_error()
    for over in (dict(M=0, rows_per_chunk=0), dict(N=0), dict(K=0)):
        base = dict(plan=None, n_tiles=0, M=256, N=256, K=512, world=2, rank=0, rows_per_chunk=128,
                    bm=128, bn=128, a=16, b=32, b_layout=tlc.B_KN, partials=48, sig=64, epoch=1,
                    land=tlc.LAND_NONE)
        base.update(over)
        r = tlc.RSArgs(**base)
        assert tlc.lib().tlc_gemm_rs(C.byref(r), None, None, 0) == tlc.ERR_INVALID_ARG, over
        assert tlc.last_error()
    E, k, N = 8, 2, 128
    a = tlc.MoERouteArgs(logits=16, tokens_per_chunk=0, world=2, rank=0, experts=E, topk=k, N=N,
                         bm=128, bn=128, order=1, topk_idx=16, gates=16, counts=16, offsets=16,
                         row_token=16, slot=16, plan=16, plan_cap=16, n_tiles_dev=16,
                         workspace=4096, x=None, x_src=None, H=64, sig=None, epoch=1)
    assert tlc.lib().tlc_moe_route(C.byref(a), None) == tlc.ERR_INVALID_ARG
    assert "tokens_per_chunk" in tlc.last_error(), tlc.last_error()


def test_gemm_ar_argument_errors():
    rs = tlc.RSArgs(plan=None, n_tiles=0, M=256, N=256, K=512, world=2, rank=0, rows_per_chunk=128,
                    bm=128, bn=128, a=16, b=32, b_layout=tlc.B_KN, partials=48, sig=64, epoch=1,
                    land=tlc.LAND_NONE)
    for over, want in [(dict(world=17, M=17 * 128), "2 * world"), (dict(), "c NULL")]:
        r = tlc.RSArgs.from_buffer_copy(rs)
        for k, v in over.items():
            setattr(r, k, v)
        args = tlc.ARArgs(r, None, None, 0)
        assert tlc.lib().tlc_gemm_ar(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG
        assert want in tlc.last_error(), tlc.last_error()
    # landing without the peers' reduced slices
    r = tlc.RSArgs.from_buffer_copy(rs)
    r.land = tlc.LAND_MEMCPY
    args = tlc.ARArgs(r, None, 128, 0)
    assert tlc.lib().tlc_gemm_ar(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG
    assert "gathered_src" in tlc.last_error()


def test_moe_route_landing_argument_errors():
    """The routing's co-located landing is validated on the host before anything
    is enqueued (no GPU is touched: every case fails its checks)."""
    T, E, k, N = 64, 8, 2, 128
    cap = tlc.moe_plan_capacity(T, k, E, N, 128, 128)

    def args(**over):
        base = dict(logits=16, tokens_per_chunk=32, world=2, rank=0, experts=E, topk=k, N=N, bm=128,
                    bn=128, order=1, topk_idx=16, gates=16, counts=16, offsets=16, row_token=16,
                    slot=16, plan=16, plan_cap=cap, n_tiles_dev=16, workspace=4096, x=None,
                    x_src=None, H=64, sig=None, epoch=1)
        base.update(over)
        return tlc.MoERouteArgs(**base)

    src = (C.c_void_p * 2)(8192, 16384)
    srcp = C.cast(src, C.POINTER(C.c_void_p))
    for over, want, text in [
        (dict(x_src=srcp), tlc.ERR_INVALID_ARG, "needs x and sig"),
        (dict(x_src=srcp, x=4096), tlc.ERR_INVALID_ARG, "needs x and sig"),
        (dict(x_src=srcp, x=4096, sig=64, H=60), tlc.ERR_UNSUPPORTED, "H % 8"),
        (dict(x_src=srcp, x=4096, sig=64, epoch=0), tlc.ERR_INVALID_ARG, "epoch"),
        (dict(x_src=srcp, x=4104, sig=64), tlc.ERR_MISALIGNED, "16-byte"),
    ]:
        a = args(**over)
        assert tlc.lib().tlc_moe_route(C.byref(a), None) == want, (over, tlc.last_error())
        assert text in tlc.last_error(), tlc.last_error()


def test_plan_capacity_and_query():
    d = tlc.PlanDesc(tlc.MODE_AG, 8, 3, 8192, 3200, 1024, 256, 256, tlc.ORDER_RANK_OFFSET, 4)
    n = C.c_int64(0)
    assert tlc.lib().tlc_chunk_plan(C.byref(d), None, 0, C.byref(n), None) == 0
    assert n.value == 32 * 13
    tiles = (tlc.Tile * 10)()
    assert tlc.lib().tlc_chunk_plan(C.byref(d), tiles, 10, C.byref(n), None) == tlc.ERR_CAPACITY
    bad = tlc.PlanDesc(tlc.MODE_AG, 8, 8, 8192, 3200, 1024, 256, 256, 1, 1)
    assert tlc.lib().tlc_chunk_plan(C.byref(bad), None, 0, C.byref(n), None) == tlc.ERR_INVALID_ARG
    bad = tlc.PlanDesc(tlc.MODE_AG, 8, 0, 8190, 3200, 1024, 256, 256, 1, 1)
    assert tlc.lib().tlc_chunk_plan(C.byref(bad), None, 0, C.byref(n), None) == tlc.ERR_INVALID_ARG
    bad = tlc.PlanDesc(tlc.MODE_MOE, 8, 0, 8192, 3200, 1024, 256, 256, 1, 1)
    assert tlc.lib().tlc_chunk_plan(C.byref(bad), None, 0, C.byref(n), None) == tlc.ERR_INVALID_ARG
    bad = tlc.PlanDesc(tlc.MODE_AG, 8, 0, 8192, 3200, 1024, 256, 256, 1, 1, 256, 0)
    assert tlc.lib().tlc_chunk_plan(C.byref(bad), None, 0, C.byref(n), None) == tlc.ERR_INVALID_ARG
    bad = tlc.PlanDesc(tlc.MODE_AG, 8, 0, 8192, 3200, 1024, 256, 256, 1, 1, 4, -1)
    assert tlc.lib().tlc_chunk_plan(C.byref(bad), None, 0, C.byref(n), None) == tlc.ERR_INVALID_ARG
    # split: 52 tiles per chunk, chunks at key >= 6 split four ways -> +2 * 52 * 3 units
    d = tlc.PlanDesc(tlc.MODE_AG, 8, 3, 8192, 3200, 1024, 256, 256, tlc.ORDER_RANK_OFFSET, 4, 4, 6)
    assert tlc.lib().tlc_chunk_plan(C.byref(d), None, 0, C.byref(n), None) == 0
    assert n.value == 32 * 13 + 2 * 52 * 3


def test_split_workspace_bytes():
    assert tlc.split_workspace_bytes(0, 4, 256, 256) == 0
    assert tlc.split_workspace_bytes(10, 1, 256, 256) == 0
    assert tlc.split_workspace_bytes(10, 4, 256, 256) == 10 * (256 + 4 * 256 * 256 * 4)
    assert tlc.split_workspace_bytes(3, 2, 128, 128) == 3 * (256 + 2 * 128 * 128 * 4)


def test_moe_sizes():
    assert tlc.moe_plan_capacity(4096, 8, 64, 768, 256, 256) == (4096 * 8 // 256 + 64) * 3
    assert tlc.moe_workspace_bytes(4096, 8, 64, 256) >= 4096 * 8 + 65 * 4 + 2 * 192 * 4
    assert tlc.moe_plan_capacity(0, 8, 64, 768, 256, 256) == 0


def test_signals_block_layout():
    # 256 words of flags, counters and status, then the epoch table
    assert C.sizeof(tlc.SignalsBlock) == (256 + tlc.EPOCH_MAX) * 4
    assert tlc.SignalsBlock.dest_done.offset == 70 * 4
    assert tlc.SignalsBlock.dest_ready.offset == 102 * 4
    assert tlc.SignalsBlock.epoch_table.offset == 256 * 4
    assert tlc.lib().tlc_signals_rewind(None, None) == tlc.ERR_INVALID_ARG
    assert tlc.lib().tlc_read_signals(None, None, None) == tlc.ERR_INVALID_ARG


def _src2():
    src = (C.c_void_p * 2)(4096, 8192)
    return C.cast(src, C.POINTER(C.c_void_p)), src


@pytest.mark.parametrize("land", [tlc.LAND_MEMCPY, tlc.LAND_COPY_ENGINE, tlc.LAND_CU])
def test_ag_grid_that_leaves_no_cus_for_the_landing_is_refused(land):
    """A copy-stream landing needs 32 CUs that no GEMM workgroup holds: a caller
    grid above 256 - 32 is refused on the host, before any device call."""
    srcp, keep = _src2()
    streams = (C.c_void_p * 1)(None)
    args = _ag_args(a=16, b=32, c=48, sig=64, land=land, a_src=srcp, grid=225)
    assert tlc.lib().tlc_ag_gemm(C.byref(args), None, streams, 1) == tlc.ERR_INVALID_ARG
    assert "compute units free" in tlc.last_error(), tlc.last_error()
    # the largest grid the host allows passes this check (and only then needs the device)
    args = _ag_args(a=16, b=32, c=48, sig=64, land=land, a_src=srcp, grid=224)
    s = tlc.lib().tlc_ag_gemm(C.byref(args), None, streams, 1)
    assert s != tlc.ERR_INVALID_ARG or "compute units free" not in tlc.last_error()
    # the co-located landing runs inside the GEMM and reserves nothing
    args = _ag_args(a=16, b=32, c=48, sig=64, land=tlc.LAND_COLOCATED, a_src=srcp, grid=256)
    s = tlc.lib().tlc_ag_gemm(C.byref(args), None, None, 0)
    assert "compute units free" not in tlc.last_error()
    args = _ag_args(a=16, b=32, c=48, sig=64, grid=-1)
    assert tlc.lib().tlc_ag_gemm(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG


def _rs_args(**over):
    base = dict(plan=16, n_tiles=4, M=256, N=256, K=512, world=2, rank=0, rows_per_chunk=128,
                bm=128, bn=128, a=16, b=32, b_layout=tlc.B_KN, partials=48, out=4096, sig=64,
                epoch=1, land=tlc.LAND_NONE)
    base.update(over)
    return tlc.RSArgs(**base)


def test_gemm_rs_send_and_grid_argument_errors():
    landing = (C.c_void_p * 2)(None, 8192)
    lp = C.cast(landing, C.POINTER(C.c_void_p))
    dst = (C.c_void_p * 2)(None, 12288)
    dp = C.cast(dst, C.POINTER(C.c_void_p))
    bad_dst = (C.c_void_p * 2)(None, 12290)
    streams = (C.c_void_p * 1)(None)
    for over, want, text in [
        (dict(send_dst=dp, send_land=9), tlc.ERR_INVALID_ARG, "send_land"),
        (dict(send_dst=dp, send_land=tlc.LAND_COLOCATED), tlc.ERR_INVALID_ARG, "send_land"),
        (dict(send_dst=C.cast(bad_dst, C.POINTER(C.c_void_p)), send_land=tlc.LAND_MEMCPY),
         tlc.ERR_INVALID_ARG, "send_dst[1]"),
        (dict(send_dst=dp, send_land=tlc.LAND_CU, n_tiles=0), tlc.ERR_INVALID_ARG, "CU sends"),
        (dict(send_dst=dp, send_land=tlc.LAND_CU, grid=225), tlc.ERR_INVALID_ARG,
         "compute units free"),
        (dict(land=tlc.LAND_CU, remote_src=lp, grid=240), tlc.ERR_INVALID_ARG,
         "compute units free"),
    ]:
        args = _rs_args(landing=lp, **over)
        s = tlc.lib().tlc_gemm_rs(C.byref(args), None, streams, 1)
        assert s == want, (over, tlc.last_error())
        assert text in tlc.last_error(), tlc.last_error()
    # GEMM-AllReduce takes no sends
    r = _rs_args(landing=lp, send_dst=dp, send_land=tlc.LAND_MEMCPY)
    args = tlc.ARArgs(r, None, 128, 0)
    assert tlc.lib().tlc_gemm_ar(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG
    assert "send_dst" in tlc.last_error()


def test_ag_moe_grid_and_topk_errors():
    srcp, keep = _src2()
    streams = (C.c_void_p * 1)(None)

    def args(**over):
        base = dict(plan=16, n_tiles_dev=16, plan_cap=100, row_token=16, tokens_per_chunk=32,
                    world=2, rank=0, experts=8, topk=2, H=64, N=128, bm=128, bn=128, x=4096,
                    x_src=srcp, w=8192, w_layout=tlc.B_KN, y=12288, sig=64, epoch=1,
                    land=tlc.LAND_MEMCPY, grid=0)
        base.update(over)
        return tlc.MoEArgs(**base)

    # H = 64: one K step, so the 8-wavefront kernel, which fills its CUs: the
    # memcpy landing keeps 32 CUs free; the CU landing always does
    for over, want, text in [(dict(grid=230), tlc.ERR_INVALID_ARG, "compute units free"),
                             (dict(H=128, land=tlc.LAND_CU, grid=230), tlc.ERR_INVALID_ARG,
                              "compute units free"),
                             (dict(topk=9), tlc.ERR_UNSUPPORTED, "topk"),
                             (dict(plan_cap=-1), tlc.ERR_INVALID_ARG, "plan_cap")]:
        a = args(**over)
        assert tlc.lib().tlc_ag_moe(C.byref(a), None, streams, 1) == want, (over, tlc.last_error())
        assert text in tlc.last_error(), tlc.last_error()
    # H = 128 (even number of K steps): the whole-tile kernel shares its CUs with
    # the runtime's copies, so a grid of every CU passes the host check
    a = args(H=128, grid=256)
    s = tlc.lib().tlc_ag_moe(C.byref(a), None, streams, 1)
    assert "compute units free" not in tlc.last_error(), tlc.last_error()


def test_moe_route_static_refuses_oversize_on_the_host():
    """The routing variant without allocation refuses a problem whose workspace
    exceeds its static array, before any device call."""
    assert tlc.moe_static_workspace_bytes() == 4 << 20
    T, E, k = 1 << 20, 64, 16
    need = tlc.moe_workspace_bytes(T, k, E, 128)
    assert need > tlc.moe_static_workspace_bytes()
    a = tlc.MoERouteArgs(logits=16, tokens_per_chunk=T // 8, world=8, rank=0, experts=E, topk=k,
                         N=128, bm=128, bn=128, order=1, topk_idx=16, gates=16, counts=16,
                         offsets=16, row_token=16, slot=16, plan=16,
                         plan_cap=tlc.moe_plan_capacity(T, k, E, 128, 128, 128), n_tiles_dev=16,
                         workspace=None, x=None, x_src=None, H=64, sig=None, epoch=1)
    assert tlc.lib().tlc_moe_route_static(C.byref(a), None) == tlc.ERR_CAPACITY
    assert "static one holds" in tlc.last_error(), tlc.last_error()
    assert tlc.lib().tlc_moe_route_static(None, None) == tlc.ERR_INVALID_ARG


def test_streamk_schedule_accepted_and_sized():
    """TLC_SCHED_STREAMK passes the schedule check (the call then fails on its NULL
    operands, not on the schedule), and its workspace query covers any grid."""
    args = _ag_args(schedule=tlc.SCHED_STREAMK)
    assert tlc.lib().tlc_ag_gemm(C.byref(args), None, None, 0) == tlc.ERR_INVALID_ARG
    assert "schedule" not in tlc.last_error(), tlc.last_error()
    block = 256 + 4 * 256 * 256 * 4
    assert tlc.streamk_workspace_bytes(0) == 256 * block
    assert tlc.streamk_workspace_bytes(1) == block
