"""GEMM-AllReduce on the GPU (through the C ABI) against the float64 oracle:
the scatter-order GEMM, the reduce of this rank's slice, and the all-gather of
the peers' reduced slices into the M x N output.  Every rank on small shapes
with ragged tiles, every landing backend, integer inputs bit for bit; the
4096 x 4096 x 2048 tensor-parallel shape in full."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import gemm as og
from tests.parity import absmax_bf16, check_close, check_exact, log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import ARProblem
else:  # collected on CPU-only hosts, never run there
    from tile_level_communication_amd import tlc  # noqa: F401

LANDS = {"none": 0, "copy_engine": 1, "cu": 2, "memcpy": 3, "colocated": 4}

SHAPES = [
    ("w2_256x256x512_t128", 2, 128, 512, 256, 128),
    ("w4_ragged_400x264x192_t256", 4, 100, 192, 264, 256),
    ("w3_ragged_600x392x320_t128", 3, 200, 320, 392, 128),
    # whole-tile kernel (M % 256 == 0, an even number of K steps) with a last
    # column tile of 8: one wavefront column stores nothing
    ("w2_whole_512x264x256_t256", 2, 256, 256, 264, 256),
]


def _run(inp, W, rank, tile, layout, land, copy_wgs=0, **kw):
    prob = ARProblem(inp.a, inp.b, inp.remote, inp.gathered, W, rank, tile, tile, layout, **kw)
    if land == 0:
        prob.place_all()
    else:
        prob.poison_remote()
    prob.run(land, copy_wgs=copy_wgs)
    torch.cuda.synchronize()
    st = prob.sig.read_status()
    assert st[0] == 0, f"device status {st}"
    return prob, prob.partials.cpu().numpy(), prob.c.cpu().numpy()


@pytest.mark.parametrize("land", list(LANDS))
@pytest.mark.parametrize("layout", [0, 1], ids=["KN", "NK"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_ar_small_parity(shape, layout, land):
    name, W, R, K, N, tile = shape
    for integer in (False, True):
        for rank in range(W):
            log(f"[ar] {name} layout={layout} land={land} int={integer} rank={rank}")
            inp = si.ar_inputs(400 + W, W, rank, R, N, K, remote_std=0.5, integer=integer)
            p_ref, c_ref = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, W, rank)
            _, p, c = _run(inp, W, rank, tile, layout, LANDS[land])
            if integer:
                check_exact(p, p_ref, name + " partials")
                check_exact(c, c_ref, name + " all-reduced")
            else:
                am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
                check_close(p, p_ref, K, am, bm, name + " partials")
                check_close(c, c_ref, K, am, bm, name + " all-reduced")
                # the gathered rows are copies: bit for bit
                for ch in range(W):
                    if ch != rank:
                        rows = c[ch * R:(ch + 1) * R]
                        assert np.array_equal(rows.view(np.uint32), inp.gathered[ch].view(np.uint32))


@pytest.mark.parametrize("land", ["memcpy", "cu", "colocated"])
def test_ar_fresh_data_every_call(land):
    """The peers' partials and reduced slices change between calls and the
    landing targets are poisoned before each call."""
    W, R, K, N, rank = 4, 128, 256, 256, 2
    inps = [si.ar_inputs(420 + i, W, rank, R, N, K, remote_std=0.5) for i in range(2)]
    for i in (1,):
        inps[i].a[:] = inps[0].a
        inps[i].b[:] = inps[0].b
    prob = ARProblem(inps[0].a, inps[0].b, inps[0].remote, inps[0].gathered, W, rank, 128, 128)
    for it, inp in enumerate([inps[0], inps[1], inps[0], inps[1]]):
        log(f"[ar fresh] land={land} iteration={it}")
        for s in range(W):
            if s != rank:
                prob.remote_src[s].copy_(torch.from_numpy(inp.remote[s]))
                prob.gathered_src[s].copy_(torch.from_numpy(inp.gathered[s]))
        prob.poison_remote()
        prob.run(LANDS[land])
        torch.cuda.synchronize()
        assert prob.sig.read_status()[0] == 0
        _, c_ref = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, W, rank)
        check_close(prob.c.cpu().numpy(), c_ref, K, absmax_bf16(inp.a), absmax_bf16(inp.b), f"iter{it}")


def test_ar_colocated_copy_workgroups():
    """Co-located all-gather: any number of copying workgroups, any grid, gives
    the same bits, and a copy-only call (no units) fills C's other chunks."""
    W, R, K, N, rank = 3, 96, 128, 200, 1
    inp = si.ar_inputs(430, W, rank, R, N, K, remote_std=0.5)
    _, c_ref = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, W, rank)
    outs = []
    for grid, cw in ((0, 0), (1, 1), (5, 3), (16, 16)):
        log(f"[ar coloc] grid={grid} copy_wgs={cw}")
        prob = ARProblem(inp.a, inp.b, inp.remote, inp.gathered, W, rank, 128, 128)
        for call in range(2):
            prob.poison_remote()
            prob.run(tlc.LAND_COLOCATED, grid=grid, copy_wgs=cw)
            torch.cuda.synchronize()
            assert prob.sig.read_status()[0] == 0
            outs.append(prob.c.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    check_close(outs[0], c_ref, K, absmax_bf16(inp.a), absmax_bf16(inp.b), "coloc")
    log("[ar coloc] copy-only call")
    prob.poison_remote()
    n = prob.n_tiles
    prob.n_tiles = 0
    prob.run(tlc.LAND_COLOCATED, copy_wgs=2)
    prob.n_tiles = n
    torch.cuda.synchronize()
    assert prob.sig.read_status()[0] == 0
    c = prob.c.cpu().numpy()
    for ch in range(W):
        if ch != rank:
            assert np.array_equal(c[ch * R:(ch + 1) * R].view(np.uint32), inp.gathered[ch].view(np.uint32))


@pytest.mark.parametrize("rank", [0, 3])
def test_ar_4096_full_size(rank):
    wl = si.WORKLOADS[1]
    log(f"[ar full] 4096x4096x2048 w4 rank={rank}: generating inputs")
    inp = si.ar_inputs(1, wl.world, rank, wl.rows_per_chunk, wl.n, wl.k, wl.a_std, wl.b_std,
                       wl.remote_std)
    p_ref, c_ref = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, wl.world, rank)
    am, bm = absmax_bf16(inp.a), absmax_bf16(inp.b)
    for land in ("memcpy", "colocated"):
        log(f"[ar full] rank={rank}: {land} landing")
        _, p, c = _run(inp, wl.world, rank, 256, tlc.B_KN, LANDS[land])
        check_close(p, p_ref, wl.k, am, bm, "partials")
        check_close(c, c_ref, wl.k, am, bm, "all-reduced")


@pytest.mark.parametrize("land", ["memcpy", "colocated"])
@pytest.mark.parametrize("sched", ["dynamic", "static"])
def test_ar_split_parity(land, sched):
    """GEMM-AllReduce with tiles split along K (partial slots, in-order fixup):
    integer inputs bit for bit, with the all-gather landed or co-located."""
    schedule = tlc.SCHED_DYNAMIC if sched == "dynamic" else tlc.SCHED_STATIC
    for (name, W, R, K, N, tile) in SHAPES:
        rank = W - 1
        log(f"[ar split] {name} land={land} sched={sched}")
        inp = si.ar_inputs(440 + W, W, rank, R, N, K, integer=True)
        p_ref, c_ref = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, W, rank)
        _, p, c = _run(inp, W, rank, tile, tlc.B_KN, LANDS[land], split_k=3, split_from=0,
                       schedule=schedule)
        check_exact(p, p_ref, name + " partials")
        check_exact(c, c_ref, name + " all-reduced")
