"""AG-MoE on the GPU (through the C ABI) against the oracle: routing arrays and
the readiness-sorted tile list bit for bit, gates within 1e-6, the grouped GEMM
within the GEMM tolerance (integer inputs bit for bit)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import moe as om
from oracle import plan as op
from tests.parity import absmax_bf16, check_close, check_exact, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import LAND_WITH_ROUTE, MoEProblem
else:  # collected on CPU-only hosts, never run there
    LAND_WITH_ROUTE = -1

# "route": the routing's top-k kernel lands the chunks, the GEMM waits for the flags
LANDS = {"none": 0, "copy_engine": 1, "cu": 2, "memcpy": 3, "colocated": 4, "route": LAND_WITH_ROUTE}


def _check_routing(prob, ref, order):
    np.testing.assert_array_equal(prob.topk_idx.cpu().numpy(), ref["topk"])
    np.testing.assert_array_equal(prob.counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(prob.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(prob.row_token.cpu().numpy(), ref["row_token"])
    np.testing.assert_array_equal(prob.slot.cpu().numpy(), ref["slot"])
    g = prob.gates.cpu().numpy().astype(np.float64)
    assert np.abs(g - ref["gates"]).max() <= 1e-6
    n = int(prob.n_tiles_dev.cpu().item())
    want = op.moe_plan(ref["counts"], ref["offsets"], ref["row_token"], prob.Tc, prob.world, prob.rank,
                       prob.N, prob.bm, prob.bn, order)
    got = prob.plan[:n].cpu().numpy().astype(np.int64)
    got[:, 5] &= 0xFFFFFFFF
    assert n == len(want)
    np.testing.assert_array_equal(got, np.array(want, dtype=np.int64))


SMALL = [
    # name, W, Tc, H, N, E, k, tile
    ("w4_t64_e16_k4_h128_n136_t128", 4, 16, 128, 136, 16, 4, 128),
    ("w2_t80_e64_k8_h192_n256_t256", 2, 40, 192, 256, 64, 8, 256),
    ("w8_t256_e8_k2_h64_n512_t128", 8, 32, 64, 512, 8, 2, 128),
    # the whole-tile kernel (256 tiles, H / 64 even) on ragged experts, with a
    # last column tile of 136: one wavefront column of each unit stores 8 columns
    ("w4_t96_e16_k4_h256_n392_t256", 4, 24, 256, 392, 16, 4, 256),
]


@pytest.mark.parametrize("land", list(LANDS))
@pytest.mark.parametrize("layout", [0, 1], ids=["KN", "NK"])
@pytest.mark.parametrize("shape", SMALL, ids=[s[0] for s in SMALL])
def test_moe_small_parity(shape, layout, land):
    name, W, Tc, H, N, E, k, tile = shape
    for integer in (False, True):
        inp = si.moe_inputs(300 + W, W, Tc, H, N, E, integer=integer)
        for rank in sorted({0, W - 1, W // 2}):
            for order in (tlc.ORDER_RANK_OFFSET, tlc.ORDER_NATURAL):
                log(f"[moe] {name} layout={layout} land={land} int={integer} rank={rank} order={order}")
                ref = om.route(inp.logits, k, W, rank, Tc)
                prob = MoEProblem(inp.x_chunks, inp.logits, inp.w, rank, k, tile, tile, layout, order)
                if LANDS[land] == 0:
                    prob.place_all()
                else:
                    prob.poison_remote()
                prob.run(LANDS[land])
                torch.cuda.synchronize()
                assert prob.sig.read_status()[0] == 0
                _check_routing(prob, ref, order)
                y_ref = om.grouped_gemm(inp.x_chunks, inp.w, ref["offsets"], ref["row_token"])
                y = prob.y.cpu().numpy()
                if integer:
                    check_exact(y, y_ref, name)
                else:
                    check_close(y, y_ref, H, absmax_bf16(inp.x_chunks), absmax_bf16(inp.w), name)


def test_moe_ties_route_to_lower_expert():
    W, Tc, H, N, E, k = 2, 32, 64, 128, 16, 4
    inp = si.moe_inputs(320, W, Tc, H, N, E)
    inp.logits[:] = np.round(inp.logits * 2) / 2      # many exact ties
    log("[moe ties]")
    ref = om.route(inp.logits, k, W, 1, Tc)
    prob = MoEProblem(inp.x_chunks, inp.logits, inp.w, 1, k, 128, 128)
    prob.poison_remote()
    prob.run(tlc.LAND_COPY_ENGINE)
    torch.cuda.synchronize()
    _check_routing(prob, ref, tlc.ORDER_RANK_OFFSET)


def test_moe_route_long_block_scan():
    """16500 tokens in 4 chunks of 4125: each chunk is cut into 258 blocks of
    up to 16 tokens (the last of 13), 1032 blocks in all, so each of the plan
    kernel's sixteen wavefronts takes a run of 65 blocks and reads its counts
    twice (the path runs of up to 16 blocks do not take)."""
    W, Tc, H, N, E, k = 4, 4125, 64, 128, 16, 2
    inp = si.moe_inputs(321, W, Tc, H, N, E)
    log("[moe long scan] T=16500")
    ref = om.route(inp.logits, k, W, 2, Tc)
    prob = MoEProblem(inp.x_chunks, inp.logits, inp.w, 2, k, 256, 256)
    prob.route()
    torch.cuda.synchronize()
    _check_routing(prob, ref, tlc.ORDER_RANK_OFFSET)


ROUTE_EDGES = [
    # name, W, Tc, E, k, tile
    ("w1_tc70_e64_k16", 1, 70, 64, 16, 128),     # one rank, the largest k, a partial block
    ("w3_tc5_e10_k3", 3, 5, 10, 3, 256),         # chunks shorter than a block, a partial expert group
    ("w32_tc7_e33_k16", 32, 7, 33, 16, 128),     # the largest world, 33 experts
    ("w5_tc17_e1_k1", 5, 17, 1, 1, 256),         # a single expert
]


@pytest.mark.parametrize("shape", ROUTE_EDGES, ids=[s[0] for s in ROUTE_EDGES])
def test_moe_route_edge_shapes(shape):
    """The routing alone at the edges of its blocking (chunks of fewer or more
    than 16 tokens, expert counts that do not fill a group of 16, one or 32
    ranks, k = 1 and 16, one expert): every routing array and the tile list bit
    for bit, at the first and last rank, in both orders."""
    name, W, Tc, E, k, tile = shape
    inp = si.moe_inputs(340 + W, W, Tc, 64, 128, E)
    for rank in sorted({0, W - 1}):
        for order in (tlc.ORDER_RANK_OFFSET, tlc.ORDER_NATURAL):
            log(f"[moe route edge] {name} rank={rank} order={order}")
            ref = om.route(inp.logits, k, W, rank, Tc)
            prob = MoEProblem(inp.x_chunks, inp.logits, inp.w, rank, k, tile, tile, tlc.B_KN, order)
            prob.route()
            torch.cuda.synchronize()
            _check_routing(prob, ref, order)


@pytest.mark.parametrize("rank", [0, 5])
def test_moe_full_size(rank):
    wl = si.WORKLOADS[4]
    log(f"[moe full] {wl.name} rank={rank}")
    inp = si.workload_inputs(4)
    ref = om.route(inp.logits, wl.topk, wl.world, rank, wl.rows_per_chunk)
    prob = MoEProblem(inp.x_chunks, inp.logits, inp.w, rank, wl.topk, 256, 256, tlc.B_KN)
    prob.poison_remote()
    prob.run(tlc.LAND_COPY_ENGINE)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    _check_routing(prob, ref, tlc.ORDER_RANK_OFFSET)
    assert int(ref["counts"].sum()) == 4096 * 8
    y_ref = om.grouped_gemm(inp.x_chunks, inp.w, ref["offsets"], ref["row_token"])
    check_close(prob.y.cpu().numpy(), y_ref, wl.k, absmax_bf16(inp.x_chunks), absmax_bf16(inp.w),
                "moe full")
    log(f"[moe full] {wl.name} rank={rank}: co-located landing")
    prob.poison_remote()
    prob.y.fill_(float("nan"))
    prob.run(tlc.LAND_COLOCATED)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    _check_routing(prob, ref, tlc.ORDER_RANK_OFFSET)
    check_close(prob.y.cpu().numpy(), y_ref, wl.k, absmax_bf16(inp.x_chunks), absmax_bf16(inp.w),
                "moe full coloc")
    log(f"[moe full] {wl.name} rank={rank}: landing beside the routing")
    prob.poison_remote()
    prob.y.fill_(float("nan"))
    prob.run(LAND_WITH_ROUTE)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    _check_routing(prob, ref, tlc.ORDER_RANK_OFFSET)
    check_close(prob.y.cpu().numpy(), y_ref, wl.k, absmax_bf16(inp.x_chunks), absmax_bf16(inp.w),
                "moe full route landing")


@pytest.mark.parametrize("land", ["route", "colocated", "memcpy"])
def test_moe_fresh_data_each_call(land):
    """Three calls on one problem, the peers' tokens changed and the landed rows
    poisoned before each: every call must see its own call's data (flags of an
    earlier epoch do not count)."""
    W, Tc, H, N, E, k = 4, 48, 128, 256, 16, 4
    inp = si.moe_inputs(330, W, Tc, H, N, E, integer=True)
    rank = 1
    ref = om.route(inp.logits, k, W, rank, Tc)
    prob = MoEProblem(inp.x_chunks, inp.logits, inp.w, rank, k, 128, 128)
    rng = np.random.default_rng(331)
    for call in range(3):
        log(f"[moe fresh] land={land} call={call}")
        # new integer tokens for the peers (bf16 bit patterns, as the inputs are)
        x_chunks = [x if c == rank else
                    si.f32_to_bf16_bits(rng.integers(-4, 5, size=(Tc, H)).astype(np.float32))
                    for c, x in enumerate(inp.x_chunks)]
        for c in range(W):
            if c != rank:
                prob.x_src[c].copy_(torch.from_numpy(x_chunks[c].view(np.int16)).view(torch.bfloat16))
        prob.poison_remote()
        prob.y.fill_(float("nan"))
        prob.run(LANDS[land])
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        y_ref = om.grouped_gemm(x_chunks, inp.w, ref["offsets"], ref["row_token"])
        check_exact(prob.y.cpu().numpy(), y_ref, f"fresh {land} call {call}")
