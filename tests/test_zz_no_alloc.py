"""The routing entry point that allocates nothing (tlc_moe_route_static: its
workspace is a static array in device memory) against the routing with a
caller-provided workspace, through the C ABI: every output bit for bit, on
two calls in a row, the second with a smaller problem."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests.parity import log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tile_level_communication_amd import tlc
    from tile_level_communication_amd.workloads import MoEProblem


def _outputs(prob, n_tiles):
    return {"topk": prob.topk_idx.cpu().numpy(), "gates": prob.gates.cpu().numpy().view(np.uint32),
            "counts": prob.counts.cpu().numpy(), "offsets": prob.offsets.cpu().numpy(),
            "row_token": prob.row_token.cpu().numpy(), "slot": prob.slot.cpu().numpy(),
            "plan": prob.plan[:n_tiles].cpu().numpy(), "n_tiles": n_tiles}


def test_moe_route_static_matches_workspace_routing():
    # the full AG-MoE routing (8 chunks of 512 tokens, 64 experts, top-8), then
    # a smaller one (4 chunks of 96 tokens, 24 experts, top-3)
    cases = [(4, 8, 512, 64, 8, 768, 2048), (504, 4, 96, 24, 3, 136, 64)]
    for (seed, W, Tc, E, k, N, H) in cases:
        wl_inp = si.moe_inputs(seed, W, Tc, H, N, E)
        for rank in (0, W - 1):
            log(f"[no-alloc] routing W={W} Tc={Tc} E={E} k={k} rank={rank}")
            prob = MoEProblem(wl_inp.x_chunks, wl_inp.logits, wl_inp.w, rank, k, 256, 256, tlc.B_KN)
            s = prob.streams.compute
            prob.route()
            torch.cuda.synchronize()
            n = int(prob.n_tiles_dev.item())
            want = _outputs(prob, n)
            for t in (prob.topk_idx, prob.counts, prob.offsets, prob.row_token, prob.slot,
                      prob.n_tiles_dev, prob.plan):
                t.fill_(-7)
            prob.gates.fill_(float("nan"))
            tlc.moe_route_static(prob.logits, prob.Tc, prob.world, prob.rank, prob.E, prob.k,
                                 prob.N, prob.bm, prob.bn, prob.order, prob.topk_idx, prob.gates,
                                 prob.counts, prob.offsets, prob.row_token, prob.slot, prob.plan,
                                 prob.plan_cap, prob.n_tiles_dev, s)
            torch.cuda.synchronize()
            got = _outputs(prob, int(prob.n_tiles_dev.item()))
            assert got["n_tiles"] == want["n_tiles"]
            for key in want:
                if key != "n_tiles":
                    assert np.array_equal(got[key], want[key]), key
