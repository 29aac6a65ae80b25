"""Pins for oracle.plan.

* hand-derived tile orders from the pages' ordering rules (tests/golden/plan_cases.json);
* brute-force properties over a grid of small shapes, computed row by row (each
  row's chunk is row // R, found without the oracle's chunk-range helper), so an
  off-by-one in the chunk range or a wrong sign in the position formula fails.
"""
import itertools
import json
import os

import pytest

from oracle import plan as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_cases.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_orders(case):
    tiles, landing = op.chunk_plan(case["mode"], case["world"], case["rank"], case["M"], case["N"],
                                   case["R"], case["bm"], case["bn"], case["order"], case["group_m"],
                                   case.get("sub_chunks", 0))
    assert [list(t) for t in tiles] == case["tiles"]
    assert landing == case["landing"]


def _brute_props(mode, world, rank, R, N, bm, bn, group_m):
    M = world * R
    tiles, landing = op.chunk_plan(mode, world, rank, M, N, R, bm, bn, op.ORDER_RANK_OFFSET, group_m)
    # permutation of the full tile grid, every output element covered once
    cover = [[0] * N for _ in range(M)]
    for (m0, n0, mr, nc, e, mask, key, z) in tiles:
        assert e == -1 and z == 0
        assert 0 < mr <= bm and 0 < nc <= bn and m0 % bm == 0 and n0 % bn == 0
        for i in range(m0, m0 + mr):
            for j in range(n0, n0 + nc):
                cover[i][j] += 1
        rows_chunks = {i // R for i in range(m0, m0 + mr)}
        assert mask == sum(1 << c for c in rows_chunks)
        if mode == op.AG:
            want = max((c + world - rank) % world for c in rows_chunks)
        else:
            want = min((c + 2 * world - rank - 1) % world for c in rows_chunks)
        assert key == want
    assert all(v == 1 for row in cover for v in row)
    keys = [t[6] for t in tiles]
    assert keys == sorted(keys)
    assert sorted(landing) == sorted(set(range(world)) - {rank})
    if mode == op.AG:
        # tiles reading only the local chunk come first
        local = [t for t in tiles if t[5] == (1 << rank)]
        assert tiles[:len(local)] == local
    else:
        # tiles writing only the local slice come last
        local = [t for t in tiles if t[5] == (1 << rank)]
        assert local == tiles[len(tiles) - len(local):]


@pytest.mark.parametrize("mode", [op.AG, op.RS])
@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("R,bm", [(1, 1), (63, 64), (96, 64), (128, 128), (5, 4), (7, 16)])
def test_brute_force_grid(mode, world, R, bm):
    for rank in range(world):
        for group_m in (1, 4):
            _brute_props(mode, world, rank, R, 9, bm, 4, group_m)


def test_natural_order_is_row_major():
    tiles, _ = op.chunk_plan(op.AG, 4, 2, 64, 48, 16, 16, 16, op.ORDER_NATURAL, 1)
    coords = [(t[0], t[1]) for t in tiles]
    assert coords == [(m, n) for m in range(0, 64, 16) for n in range(0, 48, 16)]


def test_rank_rotation_gives_same_tile_set():
    base = None
    for rank in range(4):
        tiles, _ = op.chunk_plan(op.AG, 4, rank, 40, 24, 10, 8, 8)
        s = sorted((t[0], t[1], t[2], t[3], t[5]) for t in tiles)
        base = base or s
        assert s == base


def test_moe_plan_brute_force():
    # 3 experts, 10 tokens in 2 chunks of 5, routing chosen by hand
    world, rank, tpc = 2, 1, 5
    row_token = [5, 9, 0, 3, 4, 6, 7, 1, 2]   # expert 0: 5,9,0 | expert 1: 3,4 | expert 2: 6,7,1,2
    counts = [3, 2, 4]
    offsets = [0, 3, 5, 9]
    tiles = op.moe_plan(counts, offsets, row_token, tpc, world, rank, N=3, bm=2, bn=2)
    # expected by hand: p(chunk 1) = 0, p(chunk 0) = 1
    #  e0 mt0 rows 0,1 tokens 5,9 -> chunks {1} key 0 ; e0 mt1 row 2 token 0 -> {0} key 1
    #  e1 mt0 rows 3,4 tokens 3,4 -> {0} key 1
    #  e2 mt0 rows 5,6 tokens 6,7 -> {1} key 0 ; e2 mt1 rows 7,8 tokens 1,2 -> {0} key 1
    want = []
    for (key, e, mt, m0, mr, mask) in [(0, 0, 0, 0, 2, 2), (0, 2, 0, 5, 2, 2), (1, 0, 1, 2, 1, 1),
                                       (1, 1, 0, 3, 2, 1), (1, 2, 1, 7, 2, 1)]:
        for nt, (n0, nc) in enumerate([(0, 2), (2, 1)]):
            want.append([m0, n0, mr, nc, e, mask, key, 0])
    assert [list(t) for t in tiles] == want


@pytest.mark.parametrize("S", [2, 4])
def test_subchunk_plan_brute(S):
    """Sub-chunks: every tile's key is the largest consume position of the
    R/S-row pieces its rows touch (found row by row), local pieces first."""
    world, rank, R, N, bm, bn = 4, 2, 8, 10, 4, 4
    M = world * R
    tiles, landing = op.chunk_plan(op.AG, world, rank, M, N, R, bm, bn, sub_chunks=S)
    P = R // S
    for (m0, n0, mr, nc, e, mask, key, z) in tiles:
        pieces = {i // P for i in range(m0, m0 + mr)}
        assert mask == sum(1 << c for c in pieces)
        assert key == max((c - rank * S) % (world * S) for c in pieces)
    assert landing == [(rank * S + i) % (world * S) for i in range(S, world * S)]
    keys = [t[6] for t in tiles]
    assert keys == sorted(keys)
