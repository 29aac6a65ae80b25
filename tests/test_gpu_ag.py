"""AllGather-GEMM on the GPU (through the C ABI) against the float64 oracle.

Small shapes span several tiles with ragged edges and a tile that straddles two
chunks; every rank; both weight layouts; all three landing modes.  Integer-
valued inputs are compared bit for bit.  The full Qwen3-32B-like FFN-up shape
(8 chunks of 1024 x 5120, weight 5120 x 3200) is compared element by element
over its whole output, for every landing and schedule the bench runs, with
normal inputs and with integer inputs.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import gemm as og
from tests.parity import absmax_bf16, check_close, check_exact, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import AGProblem
else:  # collected on CPU-only hosts, never run there
    from tile_level_communication_amd import tlc  # noqa: F401

LANDS = {"none": 0, "copy_engine": 1, "cu": 2, "memcpy": 3, "colocated": 4}

SHAPES = [
    # name, W, R, K, N, tile
    ("w2_256x256x512_t128", 2, 128, 512, 256, 128),
    ("w2_256x256x512_t256_straddle", 2, 128, 512, 256, 256),
    ("w3_ragged_600x392x320_t256", 3, 200, 320, 392, 256),
    ("w5_ragged_385x136x128_t128", 5, 77, 128, 136, 128),
    # whole-tile kernel (M % 256 == 0, an even number of K steps) with a ragged
    # last column tile of 136: one wavefront column stores 8 of its 128 columns
    ("w2_whole_512x392x256_t256", 2, 256, 256, 392, 256),
]


def _run(inp, rank, tile, layout, land, **kw):
    prob = AGProblem(inp.a_chunks, inp.b, rank, tile, tile, layout, **kw)
    if land == tlc.LAND_NONE:
        prob.place_all()
    else:
        prob.poison_remote()
    prob.run(land)
    torch.cuda.synchronize()
    st = prob.sig.read_status()
    assert st[0] == 0, f"device status {st}"
    return prob, prob.c.cpu().numpy()


@pytest.mark.parametrize("land", list(LANDS))
@pytest.mark.parametrize("layout", [0, 1], ids=["KN", "NK"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_ag_small_parity(shape, layout, land):
    name, W, R, K, N, tile = shape
    for integer in (False, True):
        inp = si.ag_inputs(100 + W, W, R, N, K, integer=integer)
        ref = og.ag_gemm(inp.a_chunks, inp.b)
        for rank in range(W):
            log(f"[ag] {name} layout={layout} land={land} int={integer} rank={rank}")
            _, c = _run(inp, rank, tile, layout, LANDS[land])
            if integer:
                check_exact(c, ref, name)
            else:
                check_close(c, ref, K, absmax_bf16(inp.a_chunks), absmax_bf16(inp.b), name)


def test_ag_tile_order_does_not_change_bits():
    W, R, K, N = 4, 160, 256, 520
    inp = si.ag_inputs(120, W, R, N, K)
    outs = []
    for order in (tlc.ORDER_NATURAL, tlc.ORDER_RANK_OFFSET):
        for group_m in (1, 4):
            for grid in (0, 1, 7):
                log(f"[ag order] order={order} group_m={group_m} grid={grid}")
                prob = AGProblem(inp.a_chunks, inp.b, 2, 128, 128, tlc.B_KN, order=order, group_m=group_m)
                prob.poison_remote()
                prob.run(tlc.LAND_COPY_ENGINE, grid=grid)
                torch.cuda.synchronize()
                assert prob.sig.read_status()[0] == 0
                outs.append(prob.c.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    check_close(outs[0], og.ag_gemm(inp.a_chunks, inp.b), K, absmax_bf16(inp.a_chunks),
                absmax_bf16(inp.b), "order")


@pytest.mark.parametrize("land", ["copy_engine", "cu", "memcpy", "colocated"])
def test_ag_fresh_data_every_call(land):
    """Landed data changes between calls (and the landing rows are poisoned
    before each call): a read of stale or not-yet-landed data fails."""
    W, R, K, N = 4, 128, 256, 256
    inp1 = si.ag_inputs(130, W, R, N, K)
    inp2 = si.ag_inputs(131, W, R, N, K)
    inp2.a_chunks[1] = inp1.a_chunks[1]  # the local chunk (rank 1) stays the same
    prob = AGProblem(inp1.a_chunks, inp1.b, 1, 128, 128)
    for it, inp in enumerate([inp1, inp2, inp1, inp2]):
        log(f"[ag fresh] land={land} iteration={it}")
        for c in range(W):
            prob.a_src[c].copy_(torch.from_numpy(inp.a_chunks[c].view(np.int16)).view(torch.bfloat16))
        prob.poison_remote()
        prob.run(LANDS[land])
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_close(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp1.b), K,
                    absmax_bf16(inp.a_chunks), absmax_bf16(inp1.b), f"iter{it}")


@pytest.mark.parametrize("sched", ["dynamic", "static"])
@pytest.mark.parametrize("split", [(2, 0), (3, 1)], ids=["s2_from0", "s3_from1"])
@pytest.mark.parametrize("land", ["copy_engine", "cu", "colocated"])
def test_ag_split_parity(land, split, sched):
    """Tiles split along K (one K range per unit, fixup in split order), both
    schedules; K = 128 with three splits leaves one unit an empty K range."""
    schedule = tlc.SCHED_DYNAMIC if sched == "dynamic" else tlc.SCHED_STATIC
    for (name, W, R, K, N, tile) in SHAPES:
        for integer in (False, True):
            inp = si.ag_inputs(160 + W, W, R, N, K, integer=integer)
            ref = og.ag_gemm(inp.a_chunks, inp.b)
            for rank in sorted({0, W - 1}):
                log(f"[ag split] {name} land={land} split={split} sched={sched} int={integer} rank={rank}")
                prob, c = _run(inp, rank, tile, tlc.B_KN, LANDS[land], split_k=split[0],
                               split_from=split[1], schedule=schedule)
                if integer:
                    check_exact(c, ref, name)
                else:
                    check_close(c, ref, K, absmax_bf16(inp.a_chunks), absmax_bf16(inp.b), name)
                # the workspace counters are back at zero: a second call is right too
                prob.poison_remote()
                prob.run(LANDS[land])
                torch.cuda.synchronize()
                assert prob.sig.read_status()[0] == 0
                c2 = prob.c.cpu().numpy()
                assert np.array_equal(c2.view(np.uint32), c.view(np.uint32))


@pytest.mark.parametrize("sched", ["dynamic", "static"])
def test_ag_split_parity_nk_weight(sched):
    """Split units with an N x K weight (its own kernel instances): three
    splits from the second key on, integer inputs, bit for bit, twice."""
    schedule = tlc.SCHED_DYNAMIC if sched == "dynamic" else tlc.SCHED_STATIC
    for (name, W, R, K, N, tile) in SHAPES:
        inp = si.ag_inputs(180 + W, W, R, N, K, integer=True)
        ref = og.ag_gemm(inp.a_chunks, inp.b)
        rank = W - 1
        log(f"[ag split nk] {name} sched={sched} rank={rank}")
        prob, c = _run(inp, rank, tile, tlc.B_NK, tlc.LAND_COPY_ENGINE, split_k=3, split_from=1,
                       schedule=schedule)
        check_exact(c, ref, name)
        prob.poison_remote()
        prob.run(tlc.LAND_COPY_ENGINE)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_exact(prob.c.cpu().numpy(), ref, name + " second call")


def test_ag_split_result_independent_of_schedule():
    """With a fixed split, the output bits do not depend on schedule, grid or
    which workgroup finished a tile's units last."""
    W, R, K, N = 4, 160, 512, 520
    inp = si.ag_inputs(170, W, R, N, K)
    outs = []
    for schedule in (tlc.SCHED_DYNAMIC, tlc.SCHED_STATIC):
        for grid in (0, 1, 3, 16):
            log(f"[ag split bits] schedule={schedule} grid={grid}")
            prob = AGProblem(inp.a_chunks, inp.b, 2, 128, 128, tlc.B_KN, split_k=4, split_from=0,
                             schedule=schedule)
            prob.poison_remote()
            prob.run(tlc.LAND_COPY_ENGINE, grid=grid)
            torch.cuda.synchronize()
            assert prob.sig.read_status()[0] == 0
            outs.append(prob.c.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    check_close(outs[0], og.ag_gemm(inp.a_chunks, inp.b), K, absmax_bf16(inp.a_chunks),
                absmax_bf16(inp.b), "split bits")


@pytest.mark.parametrize("sub", [2, 4])
@pytest.mark.parametrize("land", ["copy_engine", "cu", "colocated"])
def test_ag_subchunk_parity(land, sub):
    """Each peer chunk lands as `sub` pieces with their own flags; tiles wait
    for exactly the pieces their rows read (straddling tiles included)."""
    for (name, W, R, K, N, tile) in [("w2_256x256x512_t128", 2, 128, 512, 256, 128),
                                     ("w4_512x264x192_t256", 4, 128, 192, 264, 256),
                                     ("w8_1024x136x128_t128", 8, 128, 128, 136, 128)]:
        for integer in (False, True):
            inp = si.ag_inputs(180 + W, W, R, N, K, integer=integer)
            ref = og.ag_gemm(inp.a_chunks, inp.b)
            for rank in sorted({0, W - 1}):
                log(f"[ag sub] {name} land={land} sub={sub} int={integer} rank={rank}")
                _, c = _run(inp, rank, tile, tlc.B_KN, LANDS[land], sub_chunks=sub, split_k=2,
                            split_from=W * sub - 1)
                if integer:
                    check_exact(c, ref, name)
                else:
                    check_close(c, ref, K, absmax_bf16(inp.a_chunks), absmax_bf16(inp.b), name)


def test_ag_colocated_copy_workgroups_and_grid():
    """Co-located landing: the output bits do not depend on how many
    workgroups copy or on the grid, and consecutive calls reuse the arrival
    counters (they are back at zero after every chunk)."""
    W, R, K, N = 4, 160, 256, 520
    inp = si.ag_inputs(190, W, R, N, K)
    outs = []
    for schedule in (tlc.SCHED_DYNAMIC, tlc.SCHED_STATIC):
        for grid, cw in ((0, 0), (1, 1), (3, 2), (16, 16), (16, 5), (24, 1)):
            prob = AGProblem(inp.a_chunks, inp.b, 2, 128, 128, tlc.B_KN, schedule=schedule)
            for call in range(2):
                log(f"[ag coloc] schedule={schedule} grid={grid} copy_wgs={cw} call={call}")
                prob.poison_remote()
                prob.run(tlc.LAND_COLOCATED, grid=grid, copy_wgs=cw)
                torch.cuda.synchronize()
                assert prob.sig.read_status()[0] == 0
                outs.append(prob.c.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    check_close(outs[0], og.ag_gemm(inp.a_chunks, inp.b), K, absmax_bf16(inp.a_chunks),
                absmax_bf16(inp.b), "coloc")


def test_ag_colocated_copy_only_and_errors():
    """The copy work alone (no units) lands every chunk and raises its flag;
    more copying workgroups than the grid is an argument error."""
    W, R, K, N = 5, 96, 192, 136
    inp = si.ag_inputs(191, W, R, N, K)
    prob = AGProblem(inp.a_chunks, inp.b, 3, 128, 128, tlc.B_KN)
    want = np.concatenate([c.view(np.int16) for c in inp.a_chunks])
    for how in ("ag_gemm_no_tiles", "tlc_land"):
        log(f"[ag coloc copy-only] {how}")
        prob.poison_remote()
        if how == "tlc_land":
            prob.land_only(tlc.LAND_COLOCATED)
        else:
            n = prob.n_tiles
            prob.n_tiles = 0
            prob.run(tlc.LAND_COLOCATED, copy_wgs=3)
            prob.n_tiles = n
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        got = prob.a.view(torch.int16).cpu().numpy()
        assert np.array_equal(got, want)
        # the flags reached this epoch: a GEMM that waits on them (no landing,
        # 200 ms limit) finds every chunk ready
        tlc.ag_gemm(prob.plan, prob.n_tiles, prob.M, prob.N, prob.K, W, 3, R, 128, 128, prob.a, None,
                    prob.b, tlc.B_KN, prob.c, prob.sig, prob.epoch, tlc.LAND_NONE,
                    prob.streams.compute, None, 0, 200_000_000)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_close(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp.b), K,
                    absmax_bf16(inp.a_chunks), absmax_bf16(inp.b), how)
    with pytest.raises(RuntimeError, match="copy_wgs"):
        prob.run(tlc.LAND_COLOCATED, grid=4, copy_wgs=5)
    torch.cuda.synchronize()


def test_ag_timeout_reports_status():
    """A chunk whose flag never reaches the epoch: the kernel gives up after
    the time limit, reports TIMEOUT with the chunk, and every workgroup exits."""
    W, R, K, N = 2, 128, 128, 128
    inp = si.ag_inputs(140, W, R, N, K)
    prob = AGProblem(inp.a_chunks, inp.b, 0, 128, 128)
    prob.place_all()
    log("[ag timeout] flags left below the epoch, 2 ms limit")
    prob.run(tlc.LAND_NONE, timeout_ns=2_000_000, preset_flags=False)
    st = prob.sig.read_status(prob.streams.compute)
    assert st[0] == tlc.ERR_TIMEOUT and st[2] == 1, st
    prob.sig.clear_status()
    prob.run(tlc.LAND_NONE)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_close(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp.b), K, absmax_bf16(inp.a_chunks),
                absmax_bf16(inp.b), "after timeout")


@pytest.mark.parametrize("rank", [0, 7])
def test_ag_qwen3_ffn_up_full_size(rank):
    """The whole 8192 x 3200 output of every landing and schedule the bench runs,
    element by element against the float64 oracle (a misrouted tile anywhere
    fails), and with integer inputs bit for bit."""
    wl = si.WORKLOADS[2]
    log(f"[ag full] {wl.name} rank={rank}: generating inputs and the oracle")
    inp = si.workload_inputs(2)
    ref = og.ag_gemm(inp.a_chunks, inp.b)
    am, bm = absmax_bf16(inp.a_chunks), absmax_bf16(inp.b)
    legs = [
        ("SDMA landing, dynamic schedule", tlc.LAND_COPY_ENGINE, {}),
        # the bench's headline launch: memcpy landing, whole tiles, static slots
        ("memcpy landing, static schedule", tlc.LAND_MEMCPY, dict(schedule=tlc.SCHED_STATIC)),
        ("CU landing, static schedule", tlc.LAND_CU, dict(schedule=tlc.SCHED_STATIC)),
        ("co-located landing, static schedule", tlc.LAND_COLOCATED, dict(schedule=tlc.SCHED_STATIC)),
        ("co-located landing, dynamic schedule", tlc.LAND_COLOCATED, {}),
        ("natural order, memcpy landing", tlc.LAND_MEMCPY,
         dict(schedule=tlc.SCHED_STATIC, order=tlc.ORDER_NATURAL)),
        # the bench's SDMA plan: the last chunk's tiles split in two along K
        ("SDMA landing, split 2 from key 7", tlc.LAND_COPY_ENGINE,
         dict(split_k=2, split_from=7, schedule=tlc.SCHED_STATIC)),
        ("SDMA landing, split 4 from key 1, dynamic schedule", tlc.LAND_COPY_ENGINE,
         dict(split_k=4, split_from=1)),
        ("compute only (every chunk in place)", tlc.LAND_NONE, dict(schedule=tlc.SCHED_STATIC)),
    ]
    for what, land, kw in legs:
        log(f"[ag full] {wl.name} rank={rank}: {what}")
        prob = AGProblem(inp.a_chunks, inp.b, rank, 256, 256, tlc.B_KN, **kw)
        if land == tlc.LAND_NONE:
            prob.place_all()
        else:
            prob.poison_remote()
        prob.c.fill_(float("nan"))
        prob.run(land)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0, what
        check_close(prob.c.cpu().numpy(), ref, wl.k, am, bm, f"cfg full, {what}")
        del prob
    # integer-valued inputs: the whole output bit for bit
    log(f"[ag full] {wl.name} rank={rank}: integer inputs, full compare")
    ii = si.workload_inputs(2, integer=True)
    iref = og.ag_gemm(ii.a_chunks, ii.b)
    for what, land, kw in [("CU landing, split 4 from key 2", tlc.LAND_CU, dict(split_k=4, split_from=2)),
                           ("memcpy landing, static schedule", tlc.LAND_MEMCPY,
                            dict(schedule=tlc.SCHED_STATIC))]:
        log(f"[ag full] {wl.name} rank={rank}: integer inputs, {what}")
        prob = AGProblem(ii.a_chunks, ii.b, rank, 256, 256, tlc.B_KN, **kw)
        prob.poison_remote()
        prob.run(land)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_exact(prob.c.cpu().numpy(), iref, f"cfg full integer, {what}")
        del prob


@pytest.mark.parametrize("sub", [1, 2])
def test_ag_epoch_rewind_copy_engine(sub):
    """Copy-engine flags come from a table of TLC_EPOCH_MAX epochs: calls across
    the end of the table rewind the flags and stay correct."""
    W, R, K, N = 3, 128, 128, 256
    inp = si.ag_inputs(150, W, R, N, K)
    prob = AGProblem(inp.a_chunks, inp.b, 2, 128, 128, sub_chunks=sub)
    prob.epoch = tlc.EPOCH_MAX - 2
    prob.sig.set(W * sub, prob.epoch, prob.streams.compute)
    ref = og.ag_gemm(inp.a_chunks, inp.b)
    for it in range(4):
        log(f"[ag epoch rewind] call {it}, epoch before {prob.epoch}")
        prob.poison_remote()
        prob.run(tlc.LAND_COPY_ENGINE)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        check_close(prob.c.cpu().numpy(), ref, K, absmax_bf16(inp.a_chunks), absmax_bf16(inp.b), f"call{it}")
    assert prob.epoch == 2


def test_ag_trace_stamps():
    """The optional unit trace: one entry of six per unit -- workgroup, constant-
    rate stamps at wait start, wait end and unit end, shader-cycle stamps at wait
    end and unit end -- consistent with each other, and a clock in a plausible
    range; results unchanged."""
    W, R, K, N = 4, 256, 512, 512
    inp = si.ag_inputs(140, W, R, N, K)
    prob = AGProblem(inp.a_chunks, inp.b, 1, 256, 256, tlc.B_KN, schedule=tlc.SCHED_STATIC)
    prob.poison_remote()
    trace = torch.full((prob.n_tiles, 6), -1, dtype=torch.int64, device=prob.c.device)
    log("[ag trace]")
    prob.run(tlc.LAND_COLOCATED, trace=trace)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_close(prob.c.cpu().numpy(), og.ag_gemm(inp.a_chunks, inp.b), K, absmax_bf16(inp.a_chunks),
                absmax_bf16(inp.b), "traced")
    tr = trace.cpu().numpy()
    assert (tr[:, 0] >= 0).all() and (tr[:, 0] < 256).all()
    assert (tr[:, 1] <= tr[:, 2]).all() and (tr[:, 2] < tr[:, 3]).all()
    assert (tr[:, 4] < tr[:, 5]).all()
    mhz = (tr[:, 5] - tr[:, 4]).sum() / (tr[:, 3] - tr[:, 2]).sum() * tlc.wall_clock_khz() / 1e3
    assert 300 < mhz < 3000, mhz


def test_ag_qwen3_ffn_up_every_cu_static():
    """The launch the bench times as `full_grid.static`: the compute-only GEMM on
    every compute unit with static slots (a round of 256 tiles, then 160), the
    whole 8192 x 3200 output against the float64 oracle."""
    wl = si.WORKLOADS[2]
    inp = si.workload_inputs(2)
    ref = og.ag_gemm(inp.a_chunks, inp.b)
    prob = AGProblem(inp.a_chunks, inp.b, 0, 256, 256, tlc.B_KN, group_m=8, schedule=tlc.SCHED_STATIC)
    prob.place_all()
    prob.c.fill_(float("nan"))
    cus = torch.cuda.get_device_properties(prob.c.device).multi_processor_count
    log(f"[ag full] {wl.name}: compute only on {cus} workgroups, static slots")
    prob.run(tlc.LAND_NONE, grid=cus)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_close(prob.c.cpu().numpy(), ref, wl.k, absmax_bf16(inp.a_chunks), absmax_bf16(inp.b),
                "every CU, static")
