"""GEMM-ReduceScatter on the GPU (through the C ABI) against the float64 oracle:
all W partial chunks and the reduced local slice, every rank on small shapes
and the 4-chunk 4096 x 4096 x 2048 shape, the whole output of the long-context
FFN-down shape (131072 x 5120 x 3200, 8 chunks), integer inputs bit for bit;
the sends of the partial slices to their owners bit for bit."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import gemm as og
from tests.parity import absmax_bf16, check_close, check_exact, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import RSProblem
else:  # collected on CPU-only hosts, never run there
    from tile_level_communication_amd import tlc  # noqa: F401

LANDS = {"none": 0, "copy_engine": 1, "cu": 2, "memcpy": 3, "colocated": 4}
SEND_LANDS = {"memcpy": 3, "copy_engine": 1, "cu": 2}

SHAPES = [
    ("w2_256x256x512_t128", 2, 128, 512, 256, 128),
    ("w4_ragged_400x264x192_t256", 4, 100, 192, 264, 256),
    ("w3_ragged_600x392x320_t128", 3, 200, 320, 392, 128),
    # whole-tile kernel (M % 256 == 0, an even number of K steps) with a last
    # column tile of 8: one wavefront column stores nothing
    ("w2_whole_512x264x256_t256", 2, 256, 256, 264, 256),
]


def _run(inp, W, rank, tile, layout, land, **kw):
    prob = RSProblem(inp.a, inp.b, inp.remote, W, rank, tile, tile, layout, **kw)
    if land == 0:
        prob.place_all()
    else:
        prob.poison_remote()
    prob.run(land)
    torch.cuda.synchronize()
    st = prob.sig.read_status()
    assert st[0] == 0, f"device status {st}"
    return prob, prob.partials.cpu().numpy(), prob.out.cpu().numpy()


def _remote_max(remote):
    return max(float(np.abs(v).max()) for v in remote.values()) if remote else 0.0


@pytest.mark.parametrize("land", list(LANDS))
@pytest.mark.parametrize("layout", [0, 1], ids=["KN", "NK"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_rs_small_parity(shape, layout, land):
    name, W, R, K, N, tile = shape
    for integer in (False, True):
        for rank in range(W):
            log(f"[rs] {name} layout={layout} land={land} int={integer} rank={rank}")
            inp = si.rs_inputs(200 + W, W, rank, R, N, K, remote_std=0.5, integer=integer)
            p_ref, out_ref = og.gemm_rs(inp.a, inp.b, inp.remote, W, rank)
            _, p, out = _run(inp, W, rank, tile, layout, LANDS[land])
            if integer:
                check_exact(p, p_ref, name + " partials")
                check_exact(out, out_ref, name + " out")
            else:
                am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
                check_close(p, p_ref, K, am, bm, name + " partials")
                check_close(out, out_ref, K, am, bm, name + " out")


def test_rs_zero_remote_is_local_slice():
    W, R, K, N, rank = 4, 128, 256, 256, 2
    inp = si.rs_inputs(210, W, rank, R, N, K, remote_zero=True)
    log("[rs zero-remote]")
    prob, p, out = _run(inp, W, rank, 128, tlc.B_KN, tlc.LAND_CU)
    assert np.array_equal(out.view(np.uint32), p[rank * R:(rank + 1) * R].view(np.uint32))


def test_rs_reduce_only_matches_fused():
    W, R, K, N, rank = 4, 128, 128, 512, 1
    inp = si.rs_inputs(211, W, rank, R, N, K, remote_std=2.0)
    log("[rs reduce-only]")
    prob, p, out = _run(inp, W, rank, 128, tlc.B_KN, tlc.LAND_COPY_ENGINE)
    prob.out.zero_()
    prob.reduce_only()
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    assert np.array_equal(prob.out.cpu().numpy().view(np.uint32), out.view(np.uint32))


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_rs_4096_full_size(rank):
    wl = si.WORKLOADS[1]
    log(f"[rs full] {wl.name} rank={rank}")
    inp = si.workload_inputs(1, rank=rank)
    p_ref, out_ref = og.gemm_rs(inp.a, inp.b, inp.remote, wl.world, rank)
    prob, p, out = _run(inp, wl.world, rank, 256, tlc.B_KN, tlc.LAND_COPY_ENGINE)
    am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
    check_close(p, p_ref, wl.k, am, bm, "partials")
    check_close(out, out_ref, wl.k, am, bm, "out")
    ii = si.workload_inputs(1, rank=rank, integer=True)
    p_ref, out_ref = og.gemm_rs(ii.a, ii.b, ii.remote, wl.world, rank)
    if rank == 0:
        prob, p, out = _run(ii, wl.world, rank, 256, tlc.B_NK, tlc.LAND_CU)
        check_exact(p, p_ref, "partials int")
        check_exact(out, out_ref, "out int")
    # the bench's launch with sends: memcpy landing, static slots, every send kind
    prob = RSProblem(ii.a, ii.b, ii.remote, wl.world, rank, 256, 256, tlc.B_KN,
                     schedule=tlc.SCHED_STATIC, sends=True)
    for send in SEND_LANDS.values():
        log(f"[rs full] {wl.name} rank={rank}: integer inputs, sends {send}")
        prob.partials.fill_(float("nan"))
        for c in range(wl.world):
            if c != rank:
                prob.send_dst[c].fill_(float("nan"))
        prob.poison_remote()
        prob.run(tlc.LAND_MEMCPY, send_land=send)
        torch.cuda.synchronize()
        _check_sends(prob, p_ref, f"4096 sends {send}")
        check_exact(prob.out.cpu().numpy(), out_ref, "out int with sends")


def _check_partials_blocks(prob, a, b, K, am, bm, exact, what, rows=8192):
    """Every row block of the partial product P (M x N) against the oracle."""
    M = prob.M
    for r0 in range(0, M, rows):
        idx = np.arange(r0, min(r0 + rows, M))
        got = prob.partials[r0:r0 + len(idx)].cpu().numpy()
        ref = og.gemm_partial(a, b, idx)
        if exact:
            check_exact(got, ref, f"{what} P rows {r0}..")
        else:
            check_close(got, ref, K, am, bm, f"{what} P rows {r0}..")


@pytest.mark.parametrize("rank", [0, 7])
def test_rs_ffn_down_128k_full(rank):
    """The long-context FFN-down shape (131072 x 5120 x 3200, 8 chunks): the whole
    reduced slice and every row block of the partial product against the
    float64 oracle, for the copy-engine landing, the memcpy landing with the
    sends the bench times, and the co-located landing; integer inputs bit for
    bit (K * 16 < 2^24, so every fp32 sum is exact)."""
    wl = si.WORKLOADS[3]
    log(f"[rs 128k] {wl.name} rank={rank}: generating inputs")
    inp = si.workload_inputs(3, rank=rank)
    am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
    R = wl.rows_per_chunk
    prob = RSProblem(inp.a, inp.b, inp.remote, wl.world, rank, 256, 256, tlc.B_KN,
                     schedule=tlc.SCHED_STATIC, sends=True)
    log(f"[rs 128k] rank={rank}: oracle of the reduced slice")
    p_loc, out_ref = og.gemm_rs_rows(inp.a, inp.b, inp.remote, wl.world, rank, np.arange(R))
    del p_loc
    for what, land, send in [("copy-engine landing", tlc.LAND_COPY_ENGINE, None),
                             ("memcpy landing, memcpy sends", tlc.LAND_MEMCPY, tlc.LAND_MEMCPY),
                             ("co-located landing", tlc.LAND_COLOCATED, None)]:
        log(f"[rs 128k] rank={rank}: {what}")
        prob.poison_remote()
        prob.partials.fill_(float("nan"))
        prob.out.fill_(float("nan"))
        if send is not None:
            for c in range(wl.world):
                if c != rank:
                    prob.send_dst[c].fill_(float("nan"))
        prob.run(land, send_land=send)
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0, what
        check_close(prob.out.cpu().numpy(), out_ref, wl.k, am, bm, f"out, {what}")
        if send is not None:
            blk = prob.sig.read_block()
            assert all(v == 0 for v in blk.dest_done)
            for c in range(wl.world):
                if c != rank:
                    assert blk.dest_ready[c] == prob.epoch
                    assert torch.equal(prob.send_dst[c].view(torch.int32),
                                       prob.partials[c * R:(c + 1) * R].view(torch.int32)), c
    log(f"[rs 128k] rank={rank}: every row block of P")
    _check_partials_blocks(prob, inp.a, inp.b, wl.k, am, bm, False, "normal")
    del prob, inp, out_ref
    # integer-valued inputs: the whole slice and every block of P bit for bit
    log(f"[rs 128k] rank={rank}: integer inputs")
    ii = si.workload_inputs(3, rank=rank, integer=True)
    prob = RSProblem(ii.a, ii.b, ii.remote, wl.world, rank, 256, 256, tlc.B_KN,
                     schedule=tlc.SCHED_STATIC)
    prob.poison_remote()
    prob.run(tlc.LAND_MEMCPY)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    _, iout = og.gemm_rs_rows(ii.a, ii.b, ii.remote, wl.world, rank, np.arange(R))
    check_exact(prob.out.cpu().numpy(), iout, "integer out")
    _check_partials_blocks(prob, ii.a, ii.b, wl.k, 1.0, 1.0, True, "integer")


@pytest.mark.parametrize("sched", ["dynamic", "static"])
@pytest.mark.parametrize("split", [(2, 0), (3, 2)], ids=["s2_from0", "s3_from2"])
def test_rs_split_parity(split, sched):
    """Tiles split along K: partial slots, in-order fixup; integer inputs exact."""
    schedule = tlc.SCHED_DYNAMIC if sched == "dynamic" else tlc.SCHED_STATIC
    for (name, W, R, K, N, tile) in SHAPES:
        for integer in (False, True):
            rank = W - 1
            log(f"[rs split] {name} split={split} sched={sched} int={integer}")
            inp = si.rs_inputs(220 + W, W, rank, R, N, K, remote_std=0.5, integer=integer)
            p_ref, out_ref = og.gemm_rs(inp.a, inp.b, inp.remote, W, rank)
            _, p, out = _run(inp, W, rank, tile, tlc.B_KN, tlc.LAND_COPY_ENGINE, split_k=split[0],
                             split_from=split[1], schedule=schedule)
            if integer:
                check_exact(p, p_ref, name + " partials")
                check_exact(out, out_ref, name + " out")
            else:
                am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
                check_close(p, p_ref, K, am, bm, name + " partials")
                check_close(out, out_ref, K, am, bm, name + " out")


def _check_sends(prob, p_ref, what):
    """Every outgoing slice P[c] (c != rank) arrived whole in send_dst[c]: bit for
    bit the partial the GEMM stored, and exactly the oracle's (integer inputs);
    the per-destination counts are back at zero and the ready flags at the epoch."""
    blk = prob.sig.read_block()
    assert blk.status[0] == 0, f"{what}: device status {list(blk.status)}"
    assert all(v == 0 for v in blk.dest_done), f"{what}: dest_done {list(blk.dest_done)}"
    p = prob.partials.cpu().numpy()
    check_exact(p, p_ref, what + " partials")
    R = prob.R
    for c in range(prob.world):
        if c == prob.rank:
            continue
        assert blk.dest_ready[c] == prob.epoch, (what, c, blk.dest_ready[c], prob.epoch)
        sent = prob.send_dst[c].cpu().numpy()
        assert np.array_equal(sent.view(np.uint32), p[c * R:(c + 1) * R].view(np.uint32)), (what, c)
        check_exact(sent, p_ref[c * R:(c + 1) * R], f"{what} sent slice {c}")


@pytest.mark.parametrize("send", list(SEND_LANDS))
@pytest.mark.parametrize("order", ["rank_offset", "natural"])
def test_rs_sends(send, order):
    """Scatter mode's outgoing half: the GEMM counts each destination slice's
    stored elements and raises its ready flag when the slice is complete; the
    send stream copies the slice only then.  Partials and receive buffers are
    poisoned before every call, so a copy that ran ahead of the GEMM's stores
    fails; two calls in a row check the epoch rewind of the counts."""
    od = tlc.ORDER_RANK_OFFSET if order == "rank_offset" else tlc.ORDER_NATURAL
    for (name, W, R, K, N, tile) in SHAPES:
        for rank in range(W):
            inp = si.rs_inputs(230 + W, W, rank, R, N, K, remote_std=0.5, integer=True)
            p_ref, out_ref = og.gemm_rs(inp.a, inp.b, inp.remote, W, rank)
            prob = RSProblem(inp.a, inp.b, inp.remote, W, rank, tile, tile, tlc.B_KN, order=od,
                             sends=True)
            for call in range(2):
                log(f"[rs sends] {name} send={send} order={order} rank={rank} call={call}")
                prob.partials.fill_(float("nan"))
                for c in range(W):
                    if c != rank:
                        prob.send_dst[c].fill_(float("nan"))
                prob.poison_remote()
                prob.run(tlc.LAND_CU, send_land=SEND_LANDS[send])
                torch.cuda.synchronize()
                _check_sends(prob, p_ref, f"{name} rank {rank} call {call}")
                check_exact(prob.out.cpu().numpy(), out_ref, f"{name} out")


@pytest.mark.parametrize("sched", ["dynamic", "static"])
@pytest.mark.parametrize("layout", [tlc.B_KN, tlc.B_NK], ids=["KN", "NK"])
def test_rs_sends_split_tiles(sched, layout):
    """Split tiles: only the unit that stores the summed tile counts it in; the
    weight K x N or N x K."""
    schedule = tlc.SCHED_DYNAMIC if sched == "dynamic" else tlc.SCHED_STATIC
    for (name, W, R, K, N, tile) in SHAPES:
        rank = W - 1
        inp = si.rs_inputs(240 + W, W, rank, R, N, K, remote_std=0.5, integer=True)
        p_ref, _ = og.gemm_rs(inp.a, inp.b, inp.remote, W, rank)
        prob = RSProblem(inp.a, inp.b, inp.remote, W, rank, tile, tile, layout, split_k=3,
                         split_from=0, schedule=schedule, sends=True)
        for call in range(2):
            log(f"[rs sends split] {name} sched={sched} layout={layout} call={call}")
            prob.partials.fill_(float("nan"))
            for c in range(W):
                if c != rank:
                    prob.send_dst[c].fill_(float("nan"))
            prob.run(tlc.LAND_MEMCPY, send_land=tlc.LAND_MEMCPY)
            torch.cuda.synchronize()
            _check_sends(prob, p_ref, f"{name} split call {call}")
