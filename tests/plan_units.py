"""K-split work units: the library's own scheduling format, not the pages'.

The pages keep whole output tiles.  The library can replace each tile whose
primary key is at least ``split_from`` by ``split_k`` adjacent units, one per
K range, so that the work depending on the last chunks spreads over more
compute units.  Unit s of the f-th split tile (f counted in plan order)
carries ``split = split_k | s << 8 | f << 16``; a whole tile carries 0.

This module re-derives that format from the page-derived tile order of
``oracle.plan.chunk_plan`` so that the tests can check the library's planner
unit for unit.  It is test infrastructure and holds nothing of the method.
"""
from __future__ import annotations


def split_units(tiles, split_k: int, split_from: int):
    """Expand a whole-tile plan into K-split units (see the module docstring)."""
    if split_k < 2:
        return list(tiles)
    units = []
    f = 0
    for t in tiles:
        if t[6] >= split_from:
            for s in range(split_k):
                units.append(tuple(t[:7]) + (split_k | (s << 8) | (f << 16),))
            f += 1
        else:
            units.append(tuple(t))
    return units


def split_k_range(split: int, K: int, bk: int = 64):
    """K range [k0, k1) of a unit: the bk-wide steps [s*KT//S, (s+1)*KT//S)."""
    if split == 0:
        return 0, K
    S, s = split & 0xFF, (split >> 8) & 0xFF
    kt = K // bk
    return (s * kt // S) * bk, ((s + 1) * kt // S) * bk
