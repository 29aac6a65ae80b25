"""GEMM-ReduceScatter on the GPU (through the C ABI) against the float64 oracle:
all W partial chunks and the reduced local slice, every rank on small shapes
and the 4-chunk 4096 x 4096 x 2048 shape, sampled rows of the long-context
FFN-down shape (131072 x 5120 x 3200, 8 chunks), integer inputs bit for bit."""
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

LANDS = {"none": 0, "copy_engine": 1, "cu": 2, "memcpy": 3, "colocated": 4}

SHAPES = [
    ("w2_256x256x512_t128", 2, 128, 512, 256, 128),
    ("w4_ragged_400x264x192_t256", 4, 100, 192, 264, 256),
    ("w3_ragged_600x392x320_t128", 3, 200, 320, 392, 128),
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
    if rank == 0:
        ii = si.workload_inputs(1, rank=rank, integer=True)
        p_ref, out_ref = og.gemm_rs(ii.a, ii.b, ii.remote, wl.world, rank)
        prob, p, out = _run(ii, wl.world, rank, 256, tlc.B_NK, tlc.LAND_CU)
        check_exact(p, p_ref, "partials int")
        check_exact(out, out_ref, "out int")


@pytest.mark.parametrize("rank", [0, 7])
def test_rs_ffn_down_128k_sampled(rank):
    wl = si.WORKLOADS[3]
    log(f"[rs 128k] {wl.name} rank={rank}: generating inputs")
    inp = si.workload_inputs(3, rank=rank)
    prob = RSProblem(inp.a, inp.b, inp.remote, wl.world, rank, 256, 256, tlc.B_KN)
    prob.poison_remote()
    log(f"[rs 128k] rank={rank}: run")
    prob.run(tlc.LAND_COPY_ENGINE)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    R = wl.rows_per_chunk
    rng = np.random.default_rng(10 + rank)
    local_rows = np.unique(np.concatenate([[0, 1, 255, 256, R - 1], rng.integers(0, R, 24)]))
    p_ref, out_ref = og.gemm_rs_rows(inp.a, inp.b, inp.remote, wl.world, rank, local_rows)
    idx = torch.from_numpy(local_rows).to(prob.out.device)
    out = prob.out[idx].cpu().numpy()
    p_local = prob.partials[rank * R + idx].cpu().numpy()
    am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
    check_close(p_local, p_ref, wl.k, am, bm, "local partial rows")
    check_close(out, out_ref, wl.k, am, bm, "out rows")
    # rows of the other destinations' partial chunks
    rows = np.array([c * R + o for c in range(wl.world) for o in (0, R // 2, R - 1)])
    got = prob.partials[torch.from_numpy(rows).to(prob.out.device)].cpu().numpy()
    check_close(got, og.gemm_partial(inp.a, inp.b, rows), wl.k, am, bm, "partial rows")
    # co-located: the reduce reads the peers' partials where they are
    log(f"[rs 128k] rank={rank}: co-located landing")
    prob.out.fill_(float("nan"))
    prob.run(tlc.LAND_COLOCATED)
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    check_close(prob.out[idx].cpu().numpy(), out_ref, wl.k, am, bm, "out rows coloc")


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
