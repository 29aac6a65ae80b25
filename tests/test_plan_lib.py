"""The library's host planner (tlc_chunk_plan, C++) against the oracle's tile
order: bit-exact over a grid of shapes, ranks, orders and bands, and against the
hand-derived golden cases.  K-split units are the library's own format (the
pages keep whole tiles); they are checked against tests/plan_units.py, which
expands the oracle's page-derived order, and against hand-derived cases.  Runs
on the CPU (host code)."""
import json
import os

import numpy as np
import pytest

from oracle import plan as op
from plan_units import split_k_range, split_units
from tile_level_communication_amd import tlc

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")
CASES = (json.load(open(os.path.join(GOLDEN_DIR, "plan_cases.json")))["cases"]
         + json.load(open(os.path.join(GOLDEN_DIR, "plan_split_cases.json")))["cases"])


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
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
            ref_tiles, _ = op.chunk_plan(mode, W, rank, W * R, N, R, bm, bm, op.ORDER_RANK_OFFSET, 4)
            ref_tiles = split_units(ref_tiles, split_k, split_from)
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
                                                op.ORDER_RANK_OFFSET, 4, sub)
            ref_tiles = split_units(ref_tiles, split_k, split_from)
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


def test_split_cases_expand_the_page_order():
    """Each hand-derived split case is its page-derived order (the oracle's)
    with the split tiles expanded in place."""
    split_cases = json.load(open(os.path.join(GOLDEN_DIR, "plan_split_cases.json")))["cases"]
    for case in split_cases:
        base, landing = op.chunk_plan(case["mode"], case["world"], case["rank"], case["M"], case["N"],
                                      case["R"], case["bm"], case["bn"], case["order"], case["group_m"])
        got = split_units(base, case["split_k"], case["split_from"])
        assert [list(t) for t in got] == case["tiles"]
        assert landing == case["landing"]


@pytest.mark.parametrize("K,S,want", [
    (320, 2, [(0, 128), (128, 320)]),
    (320, 3, [(0, 64), (64, 192), (192, 320)]),
    (320, 5, [(0, 64), (64, 128), (128, 192), (192, 256), (256, 320)]),
    (5120, 4, [(0, 1280), (1280, 2560), (2560, 3840), (3840, 5120)]),
])
def test_split_k_ranges_hand_values(K, S, want):
    got = [split_k_range(S | (s << 8), K) for s in range(S)]
    assert got == want
    assert split_k_range(0, K) == (0, K)


@pytest.mark.parametrize("mode", [tlc.MODE_AG, tlc.MODE_RS])
@pytest.mark.parametrize("S,split_from", [(2, 0), (3, 1), (4, 2), (7, 3)])
def test_split_units_brute(mode, S, split_from):
    """The library's split units: its unsplit plan with each tile of key >=
    split_from replaced in place by S adjacent units whose K ranges partition
    [0, K), split-tile ordinals numbered 0, 1, ... in plan order."""
    world, rank, R, N, bm, bn, K = 4, 1, 8, 16, 8, 8, 7 * 64
    M = world * R
    base = [tuple(int(x) & 0xFFFFFFFF for x in t)
            for t in tlc.chunk_plan(mode, world, rank, M, N, R, bm, bn)[0].tolist()]
    units = [tuple(int(x) & 0xFFFFFFFF for x in t)
             for t in tlc.chunk_plan(mode, world, rank, M, N, R, bm, bn, tlc.ORDER_RANK_OFFSET, 1,
                                     S, split_from)[0].tolist()]
    i = 0
    f = 0
    for t in base:
        if t[6] >= split_from:
            group = units[i:i + S]
            assert [u[:7] for u in group] == [t[:7]] * S
            assert [u[7] & 0xFF for u in group] == [S] * S
            assert [(u[7] >> 8) & 0xFF for u in group] == list(range(S))
            assert [u[7] >> 16 for u in group] == [f] * S
            covered = []
            for u in group:
                k0, k1 = split_k_range(u[7], K)
                covered.extend(range(k0, k1))
            assert covered == list(range(K))
            i += S
            f += 1
        else:
            assert units[i] == t
            i += 1
    assert i == len(units)
