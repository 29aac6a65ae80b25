"""The stream-K tail (TLC_SCHED_STREAMK) on the GPU, through the C ABI,
against the float64 oracle: AllGather-GEMM on every landing and grids whose
tails split the last tiles into two, three and four K pieces (and grids with
no tail), GEMM-RS with and without the sends, GEMM-AR; the full 8192 x 3200 x
5120 FFN-up output; integer inputs bit for bit; the same grid twice gives the
same bits; the tiles' arrival counters are back at zero after every call."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import gemm as og
from tests.parity import absmax_bf16, check_close, check_exact, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import AGProblem, ARProblem, RSProblem
else:  # collected on CPU-only hosts, never run there
    from tile_level_communication_amd import tlc  # noqa: F401

BLOCK_BYTES = 256 + 4 * 256 * 256 * 4
LANDS = {"none": 0, "cu": 2, "memcpy": 3, "colocated": 4}

# name, W, R, K, N: M % 256 == 0 and K / 64 even (the whole-tile kernel)
SHAPES = [
    # 4 x 3 tiles (last column 136 wide), 16 K steps
    ("w2_1024x648x1024", 2, 512, 1024, 648),
    # 4 x 1 tiles, 32 K steps
    ("w4_1024x256x2048", 4, 256, 2048, 256),
]
# 12 tiles of 16 K steps: tails of 2, 4 and 3 tiles in two pieces on 5, 8
# and 9 workgroups, every tile in the tail on 24; 4 tiles of 32 steps: one
# tile in three pieces on 3, all four in three pieces on 7 and in four on 16
GRIDS = [3, 5, 7, 8, 9, 16, 24]


def _counters_zero(ws):
    hdr = ws.view(-1, BLOCK_BYTES)[:, :4].contiguous().view(torch.int32).cpu().numpy()
    return bool((hdr == 0).all())


@pytest.mark.parametrize("land", list(LANDS))
@pytest.mark.parametrize("layout", [0, 1], ids=["KN", "NK"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_streamk_ag_parity(shape, layout, land):
    name, W, R, K, N = shape
    for integer in (False, True):
        inp = si.ag_inputs(600 + W, W, R, N, K, integer=integer)
        ref = og.ag_gemm(inp.a_chunks, inp.b)
        am, bm = absmax_bf16(inp.a_chunks), absmax_bf16(inp.b)
        for rank in (0, W - 1):
            prob = AGProblem(inp.a_chunks, inp.b, rank, 256, 256, layout,
                             schedule=tlc.SCHED_STREAMK)
            for grid in GRIDS:
                log(f"[sk ag] {name} layout={layout} land={land} int={integer} rank={rank} grid={grid}")
                outs = []
                for rep in range(2):
                    if LANDS[land] == tlc.LAND_NONE:
                        prob.place_all()
                    else:
                        prob.poison_remote()
                    prob.c.fill_(float("nan"))
                    prob.run(LANDS[land], grid=grid)
                    torch.cuda.synchronize()
                    st = prob.sig.read_status()
                    assert st[0] == 0, f"device status {st}"
                    assert _counters_zero(prob.workspace), "tile counters left nonzero"
                    outs.append(prob.c.cpu().numpy())
                if integer:
                    check_exact(outs[0], ref, name)
                else:
                    check_close(outs[0], ref, K, am, bm, name)
                assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), \
                    "same grid, different bits"
            del prob


def test_streamk_ag_qwen3_ffn_up_full_size():
    """The 8192 x 3200 x 5120 FFN-up shape with the tail, the whole output
    element by element: compute only and the co-located landing on every CU
    (one round of whole tiles, then 160 tiles in three K pieces), memcpy and CU
    landings (224 workgroups: no tail, the static schedule); integer inputs bit
    for bit."""
    wl = si.WORKLOADS[2]
    log(f"[sk ag full] {wl.name}: generating inputs and the oracle")
    inp = si.workload_inputs(2)
    ref = og.ag_gemm(inp.a_chunks, inp.b)
    am, bm = absmax_bf16(inp.a_chunks), absmax_bf16(inp.b)
    for rank in (0, 5):
        prob = AGProblem(inp.a_chunks, inp.b, rank, 256, 256, tlc.B_KN, schedule=tlc.SCHED_STREAMK)
        for what, land in [("compute only", tlc.LAND_NONE), ("memcpy landing", tlc.LAND_MEMCPY),
                           ("CU landing", tlc.LAND_CU), ("co-located landing", tlc.LAND_COLOCATED)]:
            log(f"[sk ag full] rank={rank}: {what}")
            if land == tlc.LAND_NONE:
                prob.place_all()
            else:
                prob.poison_remote()
            prob.c.fill_(float("nan"))
            prob.run(land)
            torch.cuda.synchronize()
            assert prob.sig.read_status()[0] == 0, what
            assert _counters_zero(prob.workspace), what
            check_close(prob.c.cpu().numpy(), ref, wl.k, am, bm, f"stream-K full, {what}")
        del prob
    log(f"[sk ag full] {wl.name}: integer inputs")
    ii = si.workload_inputs(2, integer=True)
    iref = og.ag_gemm(ii.a_chunks, ii.b)
    prob = AGProblem(ii.a_chunks, ii.b, 3, 256, 256, tlc.B_KN, schedule=tlc.SCHED_STREAMK)
    for land in (tlc.LAND_NONE, tlc.LAND_MEMCPY):
        if land == tlc.LAND_NONE:
            prob.place_all()
        else:
            prob.poison_remote()
        prob.run(land)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_exact(prob.c.cpu().numpy(), iref, f"stream-K full integer, land {land}")


@pytest.mark.parametrize("layout", [tlc.B_KN, tlc.B_NK], ids=["KN", "NK"])
def test_streamk_rs_with_sends(layout):
    """GEMM-RS with the tail: 8 x 5 tiles (the last column 128 wide) on 9 and 16
    workgroups (tails of 4 and 8 tiles in two K pieces), the weight K x N or
    N x K; the partial product, the reduced slice and every sent slice (the
    tile that completes a destination's slice may be completed by a tail
    piece)."""
    W, R, K, N = 4, 512, 512, 1152
    for integer in (True, False):
        for rank in (0, 3):
            inp = si.rs_inputs(620, W, rank, R, N, K, remote_std=0.5, integer=integer)
            p_ref, out_ref = og.gemm_rs(inp.a, inp.b, inp.remote, W, rank)
            am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
            prob = RSProblem(inp.a, inp.b, inp.remote, W, rank, 256, 256, layout,
                             schedule=tlc.SCHED_STREAMK, sends=True)
            for grid in (9, 16):
                for send in (None, tlc.LAND_MEMCPY, tlc.LAND_CU):
                    log(f"[sk rs] layout={layout} int={integer} rank={rank} grid={grid} send={send}")
                    prob.poison_remote()
                    prob.partials.fill_(float("nan"))
                    if send is not None:
                        for c in range(W):
                            if c != rank:
                                prob.send_dst[c].fill_(float("nan"))
                    prob.run(tlc.LAND_MEMCPY, grid=grid, send_land=send)
                    torch.cuda.synchronize()
                    blk = prob.sig.read_block()
                    assert blk.status[0] == 0, list(blk.status)
                    assert _counters_zero(prob.workspace)
                    p = prob.partials.cpu().numpy()
                    out = prob.out.cpu().numpy()
                    if integer:
                        check_exact(p, p_ref, "partials")
                        check_exact(out, out_ref, "out")
                    else:
                        check_close(p, p_ref, K, am, bm, "partials")
                        check_close(out, out_ref, K, am, bm, "out")
                    if send is not None:
                        assert all(v == 0 for v in blk.dest_done), list(blk.dest_done)
                        for c in range(W):
                            if c != rank:
                                assert blk.dest_ready[c] == prob.epoch
                                sent = prob.send_dst[c].cpu().numpy()
                                assert np.array_equal(sent.view(np.uint32),
                                                      p[c * R:(c + 1) * R].view(np.uint32)), c
            del prob


def test_streamk_ar():
    """GEMM-AR with the tail (4 x 3 tiles on 5 and 9 workgroups: 2 and 3 tiles
    in two K pieces), memcpy and co-located landings."""
    W, R, K, N = 2, 512, 1024, 648
    for integer in (True, False):
        inp = si.ar_inputs(630, W, 1, R, N, K, remote_std=0.5, integer=integer)
        p_ref, c_ref = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, W, 1)
        am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
        prob = ARProblem(inp.a, inp.b, inp.remote, inp.gathered, W, 1, 256, 256, tlc.B_KN,
                         schedule=tlc.SCHED_STREAMK)
        for grid in (5, 9):
            for land in (tlc.LAND_MEMCPY, tlc.LAND_COLOCATED):
                log(f"[sk ar] int={integer} grid={grid} land={land}")
                prob.poison_remote()
                prob.run(land, grid=grid)
                torch.cuda.synchronize()
                assert prob.sig.read_status()[0] == 0
                assert _counters_zero(prob.workspace)
                p, c = prob.partials.cpu().numpy(), prob.c.cpu().numpy()
                if integer:
                    check_exact(p, p_ref, "partials")
                    check_exact(c, c_ref, "all-reduced")
                else:
                    check_close(p, p_ref, K, am, bm, "partials")
                    check_close(c, c_ref, K, am, bm, "all-reduced")
        del prob


def test_streamk_workspace_too_small_is_refused():
    W, R, K, N = 2, 512, 1024, 648
    inp = si.ag_inputs(640, W, R, N, K)
    prob = AGProblem(inp.a_chunks, inp.b, 0, 256, 256, tlc.B_KN, schedule=tlc.SCHED_STREAMK)
    prob.place_all()
    prob.workspace = prob.workspace[:BLOCK_BYTES]
    log("[sk ag] workspace of one tile for a tail of four")
    with pytest.raises(RuntimeError, match="stream-K"):
        prob.run(tlc.LAND_NONE, grid=8)
    torch.cuda.synchronize()


def test_streamk_bad_tail_tile_reported():
    """A tail tile whose plan entry lies outside the output is reported as
    BAD_PLAN with its plan index by the pieces that reach it, every workgroup
    exits, and after the status and the workspace are cleared the call with the
    plan restored is correct.  Under the tail schedule the workspace serves the
    tail only, so a plan with split units is reported as BAD_PLAN too."""
    W, R, K, N = 2, 512, 1024, 648
    inp = si.ag_inputs(650, W, R, N, K)
    ref = og.ag_gemm(inp.a_chunks, inp.b)
    prob = AGProblem(inp.a_chunks, inp.b, 0, 256, 256, tlc.B_KN, schedule=tlc.SCHED_STREAMK)
    prob.place_all()
    good = prob.plan.clone()
    # 12 tiles on 8 workgroups: tiles 8..11 form the tail, two K pieces each
    bad = 9
    prob.plan[bad, 0] = prob.M
    log("[sk ag] tail tile 9 outside the output, grid 8")
    prob.run(tlc.LAND_NONE, grid=8)
    torch.cuda.synchronize()
    st = prob.sig.read_status()
    assert st[0] == tlc.ERR_BAD_PLAN and st[1] == bad, st
    prob.sig.clear_status()
    prob.workspace.zero_()
    prob.plan.copy_(good)
    prob.run(tlc.LAND_NONE, grid=8)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    assert _counters_zero(prob.workspace)
    check_close(prob.c.cpu().numpy(), ref, K, absmax_bf16(inp.a_chunks), absmax_bf16(inp.b),
                "after a bad tail tile")
    del prob
    log("[sk ag] split units under the tail schedule, grid 8")
    prob = AGProblem(inp.a_chunks, inp.b, 0, 256, 256, tlc.B_KN, split_k=2, split_from=0,
                     schedule=tlc.SCHED_STREAMK)
    prob.place_all()
    prob.run(tlc.LAND_NONE, grid=8)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == tlc.ERR_BAD_PLAN


def test_streamk_rs_ffn_down_128k_full_with_sends():
    """The long-context FFN-down GEMM-RS (131072 x 5120 x 3200, 8 slices) with the tail
    on 240 workgroups: 42 rounds of whole tiles, then 160 tiles in three K pieces, the
    tile that completes a destination's slice possibly a tail piece.  Integer inputs
    (K * 16 < 2^24: every fp32 sum exact), so the whole partial product, the reduced
    slice and every sent slice are compared bit for bit with the oracle."""
    wl = si.WORKLOADS[3]
    rank = 0
    log(f"[sk rs 128k] {wl.name}: integer inputs")
    ii = si.workload_inputs(3, rank=rank, integer=True)
    R = wl.rows_per_chunk
    prob = RSProblem(ii.a, ii.b, ii.remote, wl.world, rank, 256, 256, tlc.B_KN,
                     schedule=tlc.SCHED_STREAMK, sends=True)
    prob.poison_remote()
    prob.partials.fill_(float("nan"))
    for c in range(wl.world):
        if c != rank:
            prob.send_dst[c].fill_(float("nan"))
    log("[sk rs 128k] memcpy landing, memcpy sends, grid 240")
    prob.run(tlc.LAND_MEMCPY, grid=240, send_land=tlc.LAND_MEMCPY)
    torch.cuda.synchronize()
    blk = prob.sig.read_block()
    assert blk.status[0] == 0, list(blk.status)
    assert all(v == 0 for v in blk.dest_done)
    assert _counters_zero(prob.workspace)
    for c in range(wl.world):
        if c != rank:
            assert blk.dest_ready[c] == prob.epoch
            assert torch.equal(prob.send_dst[c].view(torch.int32),
                               prob.partials[c * R:(c + 1) * R].view(torch.int32)), c
    log("[sk rs 128k] oracle: reduced slice and every row block of P")
    _, out_ref = og.gemm_rs_rows(ii.a, ii.b, ii.remote, wl.world, rank, np.arange(R))
    check_exact(prob.out.cpu().numpy(), out_ref, "integer out, tail")
    for r0 in range(0, prob.M, 8192):
        idx = np.arange(r0, min(r0 + 8192, prob.M))
        check_exact(prob.partials[r0:r0 + len(idx)].cpu().numpy(), og.gemm_partial(ii.a, ii.b, idx),
                    f"integer P rows {r0}.., tail")
