"""Degenerate cases on the GPU through the C ABI, against the oracle: one
rank (nothing to land, every landing mode), and a single tile smaller than the
tile shape."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import gemm as og
from oracle import moe as om
from tests.parity import absmax_bf16, check_close, check_exact, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import AGProblem, ARProblem, MoEProblem, RSProblem
else:  # collected on CPU-only hosts, never run there
    from tile_level_communication_amd import tlc  # noqa: F401

LANDS = {"none": 0, "copy_engine": 1, "cu": 2, "memcpy": 3, "colocated": 4}


@pytest.mark.parametrize("land", list(LANDS))
def test_single_rank_every_path(land):
    """world = 1: AG-GEMM is a plain GEMM, GEMM-RS's reduce is the local slice,
    GEMM-AR's output is the local product, AG-MoE routes the local tokens."""
    L = LANDS[land]
    R, K, N = 200, 128, 136
    inp = si.ag_inputs(500, 1, R, N, K, integer=True)
    log(f"[edge] W=1 AG land={land}")
    prob = AGProblem(inp.a_chunks, inp.b, 0, 128, 128, tlc.B_KN)
    prob.place_all()
    prob.run(L)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_exact(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp.b), "W=1 AG")

    rs = si.rs_inputs(501, 1, 0, R, N, K, integer=True)
    p_ref, out_ref = og.gemm_rs(rs.a, rs.b, rs.remote, 1, 0)
    log(f"[edge] W=1 RS land={land}")
    prob = RSProblem(rs.a, rs.b, rs.remote, 1, 0, 128, 128, tlc.B_KN)
    prob.run(L)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_exact(prob.partials.cpu().numpy(), p_ref, "W=1 RS partials")
    check_exact(prob.out.cpu().numpy(), out_ref, "W=1 RS out")

    ar = si.ar_inputs(502, 1, 0, R, N, K, integer=True)
    p_ref, c_ref = og.gemm_ar(ar.a, ar.b, ar.remote, ar.gathered, 1, 0)
    log(f"[edge] W=1 AR land={land}")
    prob = ARProblem(ar.a, ar.b, ar.remote, ar.gathered, 1, 0, 128, 128, tlc.B_KN)
    prob.run(L)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_exact(prob.c.cpu().numpy(), c_ref, "W=1 AR")

    mi = si.moe_inputs(503, 1, 48, 64, 72, 8, integer=True)
    ref = om.route(mi.logits, 2, 1, 0, 48)
    log(f"[edge] W=1 MoE land={land}")
    prob = MoEProblem(mi.x_chunks, mi.logits, mi.w, 0, 2, 128, 128, tlc.B_KN)
    prob.place_all()
    prob.run(L)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    assert np.array_equal(prob.row_token.cpu().numpy(), ref["row_token"])
    y_ref = om.grouped_gemm(mi.x_chunks, mi.w, ref["offsets"], ref["row_token"])
    check_exact(prob.y.cpu().numpy(), y_ref, "W=1 MoE")


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("land", ["memcpy", "colocated"])
def test_one_small_tile(tile, land):
    """A whole problem smaller than one tile (8 x 8 output, K = 64): both edges
    masked, two ranks of 4 rows each."""
    W, R, K, N = 2, 4, 64, 8
    inp = si.ag_inputs(504, W, R, N, K)
    for rank in range(W):
        log(f"[edge] tiny AG tile={tile} land={land} rank={rank}")
        prob = AGProblem(inp.a_chunks, inp.b, rank, tile, tile, tlc.B_KN)
        prob.poison_remote()
        prob.run(LANDS[land])
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_close(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp.b), K, absmax_bf16(inp.a_chunks),
                    absmax_bf16(inp.b), "tiny")


@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_ragged_last_m_tile_row_blocks(layout):
    """The 256 x 256 core skips the fragment reads and MFMAs of the 32-row
    blocks past a tile's last row (each wavefront owns four blocks; a
    wavefront with none only loads): every remainder from 1 row to a full
    tile, whole and K-split units, bit-exact against the oracle."""
    bl = tlc.B_KN if layout == "KN" else tlc.B_NK
    K, N = 192, 264
    for r in (1, 31, 32, 33, 96, 127, 128, 129, 160, 224, 255, 256):
        M = 256 + r
        inp = si.ag_inputs(505, 1, M, N, K, integer=True)
        ref = og.ag_gemm(inp.a_chunks, inp.b)
        for split in (0, 3):
            log(f"[edge] ragged M={M} layout={layout} split_k={split}")
            prob = AGProblem(inp.a_chunks, inp.b, 0, 256, 256, bl, split_k=split, split_from=0)
            prob.place_all()
            prob.run(tlc.LAND_NONE)
            torch.cuda.synchronize()
            assert prob.sig.read_status()[0] == 0
            check_exact(prob.c.cpu().numpy(), ref, f"ragged M={M} split_k={split}")


def test_bad_plan_reported_on_the_device():
    """A plan entry outside the output is caught by the GEMM before it touches
    any operand: status BAD_PLAN with the entry's plan index, every workgroup
    ends normally, and after clearing the status the same problem runs clean."""
    W, R, K, N = 2, 128, 128, 256
    inp = si.ag_inputs(160, W, R, N, K, integer=True)
    prob = AGProblem(inp.a_chunks, inp.b, 0, 128, 128, tlc.B_KN, schedule=tlc.SCHED_STATIC)
    prob.place_all()
    good = prob.plan.clone()
    bad_idx = 2
    for field, value in [(0, prob.M), (2, 129), (3, 12), (1, N)]:  # m0, m_rows, n_cols, n0
        plan = good.clone()
        plan[bad_idx, field] = value
        prob.plan = plan
        log(f"[edge] bad plan field {field} = {value}")
        prob.run(tlc.LAND_NONE)
        st = prob.sig.read_status(prob.streams.compute)
        assert st[0] == tlc.ERR_BAD_PLAN and st[1] == bad_idx, (field, st)
        prob.sig.clear_status(prob.streams.compute)
    prob.plan = good
    prob.run(tlc.LAND_NONE)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_exact(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp.b), "after bad plans")


def test_moe_tile_count_beyond_plan_capacity_reported():
    """The grouped GEMM reads its unit count from the device; a count above the
    plan capacity it was given is reported as BAD_PLAN and no unit runs."""
    mi = si.moe_inputs(504, 2, 64, 64, 128, 8, integer=True)
    prob = MoEProblem(mi.x_chunks, mi.logits, mi.w, 0, 2, 128, 128, tlc.B_KN)
    prob.place_all()
    log("[edge] MoE unit count beyond the plan capacity")
    prob.route()
    torch.cuda.synchronize()
    n = int(prob.n_tiles_dev.item())
    assert n > 1
    prob.y.fill_(7.0)
    tlc.ag_moe(prob.plan, prob.n_tiles_dev, n - 1, prob.row_token, prob.Tc, prob.world, prob.rank,
               prob.E, prob.k, prob.H, prob.N, prob.bm, prob.bn, prob.x, None, prob.w,
               prob.b_layout, prob.y, prob.sig, 0, tlc.LAND_NONE, prob.streams.compute, None, 0)
    st = prob.sig.read_status(prob.streams.compute)
    assert st[0] == tlc.ERR_BAD_PLAN and st[1] == n, st
    assert bool((prob.y == 7.0).all().item())
    prob.sig.clear_status(prob.streams.compute)


@pytest.mark.parametrize("layout", [0, 1], ids=["KN", "NK"])
def test_whole_tiles_even_and_odd_k_steps(layout):
    """Whole 256 x 256 tiles go to the kernel with only the fixed-order loop
    when the number of 64-wide K steps is even (K = 384, 5120) and to the
    general loop when it is odd (K = 320, 448); integer inputs bit for bit,
    every landing that waits."""
    bl = tlc.B_KN if layout == 0 else tlc.B_NK
    for K in (320, 384, 448):
        inp = si.ag_inputs(170 + K, 2, 256, 264, K, integer=True)
        ref = og.ag_gemm(inp.a_chunks, inp.b)
        for land in (tlc.LAND_NONE, tlc.LAND_MEMCPY, tlc.LAND_COLOCATED):
            log(f"[edge] whole tiles K={K} layout={layout} land={land}")
            prob = AGProblem(inp.a_chunks, inp.b, 1, 256, 256, bl, schedule=tlc.SCHED_STATIC)
            if land == tlc.LAND_NONE:
                prob.place_all()
            else:
                prob.poison_remote()
            prob.c.fill_(float("nan"))
            prob.run(land)
            torch.cuda.synchronize()
            assert prob.sig.read_status()[0] == 0
            check_exact(prob.c.cpu().numpy(), ref, f"whole tiles K={K}")


def test_colocated_copiers_must_fit_the_device():
    """The co-located landing is deadlock-free because its copying workgroups
    (the lowest ids) are resident before any workgroup that waits on their
    flags: a grid above the compute-unit count is fine while the copiers fit
    (bit for bit), and more copiers than compute units are refused."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    W, R, K, N = 4, 256, 256, 512
    inp = si.ag_inputs(180, W, R, N, K, integer=True)
    ref = og.ag_gemm(inp.a_chunks, inp.b)
    for sched in (tlc.SCHED_STATIC, tlc.SCHED_DYNAMIC):
        log(f"[edge] co-located grid {2 * cus} with 64 copiers, schedule {sched}")
        prob = AGProblem(inp.a_chunks, inp.b, 2, 256, 256, tlc.B_KN, schedule=sched)
        prob.poison_remote()
        prob.run(tlc.LAND_COLOCATED, grid=2 * cus, copy_wgs=64)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_exact(prob.c.cpu().numpy(), ref, "co-located, grid above the CU count")
    prob = AGProblem(inp.a_chunks, inp.b, 2, 256, 256, tlc.B_KN)
    for grid, copy_wgs in ((2 * cus, 0), (2 * cus, cus + 8)):
        with pytest.raises(tlc.TLCError) as e:
            prob.run(tlc.LAND_COLOCATED, grid=grid, copy_wgs=copy_wgs)
        assert e.value.status == tlc.ERR_INVALID_ARG and "resident" in str(e.value)
