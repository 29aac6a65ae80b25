"""The library's host planner (tlc_chunk_plan, C++) against the oracle's tile
order: bit-exact over a grid of shapes, ranks, orders and bands, and against the
hand-derived golden cases.  Runs on the CPU (host code)."""
import json
import os

import numpy as np
import pytest

from oracle import plan as op
from tile_level_communication_amd import tlc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_cases.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_library_matches_golden(case):
    tiles, landing = tlc.chunk_plan(case["mode"], case["world"], case["rank"], case["M"], case["N"],
                                    case["R"], case["bm"], case["bn"], case["order"], case["group_m"],
                                    case.get("split_k", 0), case.get("split_from", 0),
                                    case.get("sub_chunks", 0))
    assert tiles.tolist() == case["tiles"]
    assert landing == case["landing"]


@pytest.mark.parametrize("mode", [tlc.MODE_AG, tlc.MODE_RS])
@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("R,bm,bn,N", [(1, 1, 1, 3), (63, 64, 64, 130), (96, 64, 128, 256),
                                       (128, 128, 128, 512), (1024, 256, 256, 3200),
                                       (5, 4, 8, 24), (100, 256, 256, 520)])
@pytest.mark.parametrize("order", [tlc.ORDER_NATURAL, tlc.ORDER_RANK_OFFSET])
def test_library_matches_oracle(mode, world, R, bm, bn, N, order):
    M = world * R
    for rank in range(world):
        for group_m in (1, 3, 4):
            lib_tiles, lib_land = tlc.chunk_plan(mode, world, rank, M, N, R, bm, bn, order, group_m)
            ref_tiles, ref_land = op.chunk_plan(mode, world, rank, M, N, R, bm, bn, order, group_m)
            ref = np.array(ref_tiles, dtype=np.int64)
            got = lib_tiles.astype(np.int64)
            got[:, 5] &= 0xFFFFFFFF
            assert got.shape == ref.shape
            assert np.array_equal(got, ref)
            assert lib_land == ref_land


def test_full_size_plans_match_oracle():
    for (mode, W, R, N, bm) in [(tlc.MODE_RS, 8, 16384, 5120, 256), (tlc.MODE_RS, 4, 1024, 4096, 256),
                                (tlc.MODE_AG, 8, 1024, 3200, 256), (tlc.MODE_AG, 2, 128, 256, 128)]:
        for rank in (0, W - 1):
            lib_tiles, _ = tlc.chunk_plan(mode, W, rank, W * R, N, R, bm, bm, tlc.ORDER_RANK_OFFSET, 4)
            ref_tiles, _ = op.chunk_plan(mode, W, rank, W * R, N, R, bm, bm, op.ORDER_RANK_OFFSET, 4)
            assert np.array_equal(lib_tiles.astype(np.int64), np.array(ref_tiles, dtype=np.int64))


@pytest.mark.parametrize("mode", [tlc.MODE_AG, tlc.MODE_RS])
@pytest.mark.parametrize("split_k,split_from", [(2, 0), (3, 1), (4, 6), (5, 7), (255, 2)])
def test_library_split_matches_oracle(mode, split_k, split_from):
    for (W, R, N, bm) in [(8, 1024, 3200, 256), (3, 200, 392, 256), (5, 77, 136, 128)]:
        for rank in (0, W - 1):
            lib_tiles, _ = tlc.chunk_plan(mode, W, rank, W * R, N, R, bm, bm, tlc.ORDER_RANK_OFFSET, 4,
                                          split_k, split_from)
            ref_tiles, _ = op.chunk_plan(mode, W, rank, W * R, N, R, bm, bm, op.ORDER_RANK_OFFSET, 4,
                                         split_k, split_from)
            got = lib_tiles.astype(np.int64) & 0xFFFFFFFF
            ref = np.array(ref_tiles, dtype=np.int64) & 0xFFFFFFFF
            assert np.array_equal(got, ref)
            assert tlc.split_tiles(lib_tiles) == sum(1 for t in ref_tiles if (t[7] & 0xFF) >= 2 and
                                                     ((t[7] >> 8) & 0xFF) == 0)


@pytest.mark.parametrize("sub", [2, 4])
@pytest.mark.parametrize("split_k,split_from", [(0, 0), (2, 5)])
def test_library_subchunks_match_oracle(sub, split_k, split_from):
    for (W, R, N, bm) in [(8, 1024, 3200, 256), (2, 128, 256, 128), (4, 96, 136, 128)]:
        for rank in range(W):
            lib_tiles, lib_land = tlc.chunk_plan(tlc.MODE_AG, W, rank, W * R, N, R, bm, bm,
                                                 tlc.ORDER_RANK_OFFSET, 4, split_k, split_from, sub)
            ref_tiles, ref_land = op.chunk_plan(op.AG, W, rank, W * R, N, R, bm, bm,
                                                op.ORDER_RANK_OFFSET, 4, split_k, split_from, sub)
            got = lib_tiles.astype(np.int64) & 0xFFFFFFFF
            ref = np.array(ref_tiles, dtype=np.int64) & 0xFFFFFFFF
            assert np.array_equal(got, ref)
            assert lib_land == ref_land


def test_subchunk_argument_errors():
    with pytest.raises(tlc.TLCError):
        tlc.chunk_plan(tlc.MODE_RS, 4, 0, 400, 64, 100, 128, 128, sub_chunks=2)   # gather only
    with pytest.raises(tlc.TLCError):
        tlc.chunk_plan(tlc.MODE_AG, 4, 0, 400, 64, 100, 128, 128, sub_chunks=3)   # R % S
    with pytest.raises(tlc.TLCError):
        tlc.chunk_plan(tlc.MODE_AG, 8, 0, 8192, 64, 1024, 256, 256, sub_chunks=8)  # W * S > 32
