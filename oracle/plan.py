"""Oracle for the communication-aware tile order (test infrastructure only).

The method reorders the tiles of one GEMM so that work follows communication
chunks instead of the kernel's natural wave order:

* Gather mode (AllGather-GEMM): each rank starts from the chunk it already
  holds and then consumes the other chunks in increasing rank offset, i.e.
  chunk c is consumed at position p(c) = (c - rank) mod W.  DITRON paper notes,
  §3.2 (gather mode; execution starts at rank_id mod local_world_size);
  Triton-Distributed talk, swizzling section (each card handles its own data
  first while the pull of remote tiles proceeds).
* Scatter mode (GEMM-ReduceScatter): tiles whose results must leave the rank
  are produced first, the farthest destination first, and the rank's own slice
  last.  On a fully connected node every peer is one hop away; the reading
  taken here is the send position q(c) = (c - rank - 1) mod W, so destination
  rank+1 goes first and the rank itself (q = W-1) goes last.  DITRON §3.2
  (scatter mode); talk, swizzling section (compute the data the other side
  needs first, then the local part while sending).
* Non-perfect tiling: a tile whose rows straddle several chunks is keyed by
  the latest chunk it must wait for (gather mode: such tiles run after the
  fully-local ones) and, in scatter mode, by the earliest destination it feeds
  (such tiles run early).  Talk, section on non-perfect tile scheduling.
* Inside one chunk, tiles keep a locality-preserving order (group-M bands).
  AutoOverlap §5.4 / Fig. 6 and Syncopate wiki core method 5 (waves follow chunk
  completion order; intra-chunk swizzle keeps locality).
* AG-MoE: tiles of the grouped GEMM are ordered by how late their rows' data
  arrives (fewest dependencies first).  Talk, section "MoE dynamic sorting".

* Sub-chunks (AutoOverlap §6.1 inter-chunk tuning of the split factor, and
  Fig. 11(b)): each rank's chunk may arrive as S pieces, each with its own
  ready flag, so the order is the one of world*S smaller chunks.

A tile is the tuple (m0, n0, m_rows, n_cols, expert, chunk_mask, key, 0)
with ``chunk_mask`` = bit c set for every chunk c whose rows the tile reads
(gather and MoE) or writes (scatter); ``key`` = wait position / send position /
readiness used as the primary sort key.  The last field is always 0 here: the
pages keep whole tiles.
"""
from __future__ import annotations

AG, RS, MOE = 0, 1, 2
ORDER_NATURAL, ORDER_RANK_OFFSET = 0, 1


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def dense_tiles(M: int, N: int, bm: int, bn: int):
    """All (mt, nt, m0, n0, m_rows, n_cols) of an M x N output cut into bm x bn tiles."""
    out = []
    for mt in range(_ceil_div(M, bm)):
        for nt in range(_ceil_div(N, bn)):
            m0, n0 = mt * bm, nt * bn
            out.append((mt, nt, m0, n0, min(bm, M - m0), min(bn, N - n0)))
    return out


def chunk_set(m0: int, m_rows: int, rows_per_chunk: int):
    """Chunks whose rows [m0, m0 + m_rows) intersect, rows split as c*R .. (c+1)*R - 1."""
    first = m0 // rows_per_chunk
    last = (m0 + m_rows - 1) // rows_per_chunk
    return list(range(first, last + 1))


def consume_pos(c: int, world: int, rank: int) -> int:
    """Gather-mode position of chunk c: the local chunk is 0, then rank+1, rank+2, ..."""
    return (c - rank) % world


def send_pos(c: int, world: int, rank: int) -> int:
    """Scatter-mode position of destination c: rank+1 first, ..., the rank itself last."""
    return (c - rank - 1) % world


def landing_order(world: int, rank: int, n_local: int = 1):
    """Order in which the peers' chunks arrive: rank+1, rank+2, ..., rank-1 (mod W).
    With sub-chunks, `world` counts sub-chunks and the n_local ones from `rank` on
    are the local rank's own."""
    return [(rank + i) % world for i in range(n_local, world)]


def chunk_plan(mode: int, world: int, rank: int, M: int, N: int, rows_per_chunk: int,
               bm: int, bn: int, order: int = ORDER_RANK_OFFSET, group_m: int = 1,
               sub_chunks: int = 0):
    """Tile list in execution order for a dense gather (AG) or scatter (RS) GEMM.

    Sort key: (key, mt // group_m, nt, mt), where key = max consume_pos over the
    touched chunks (AG), min send_pos over the touched chunks (RS), or 0 when the
    natural (un-swizzled) order is requested.  Python's sort is stable and the
    key is total, so the order is unique.

    Sub-chunks (gather mode, AutoOverlap §6.1 / Fig. 11(b) split factor): each
    rank's chunk arrives as S pieces of R/S rows with their own flags, so chunks,
    positions and masks are those of world*S pieces, rank*S being the first local
    one; the S local pieces are the rank's own (never landed).
    """
    assert mode in (AG, RS)
    assert M == world * rows_per_chunk
    S = sub_chunks if sub_chunks and sub_chunks > 1 else 1
    if S > 1:
        assert mode == AG and rows_per_chunk % S == 0 and world * S <= 32
    n_local = S
    world, rank, rows_per_chunk = world * S, rank * S, rows_per_chunk // S
    tiles = []
    for (mt, nt, m0, n0, mr, nc) in dense_tiles(M, N, bm, bn):
        cs = chunk_set(m0, mr, rows_per_chunk)
        mask = 0
        for c in cs:
            mask |= 1 << c
        if order == ORDER_NATURAL:
            key = 0
        elif mode == AG:
            key = max(consume_pos(c, world, rank) for c in cs)
        else:
            key = min(send_pos(c, world, rank) for c in cs)
        tiles.append(((key, mt // group_m, nt, mt), (m0, n0, mr, nc, -1, mask, key, 0)))
    tiles.sort(key=lambda kv: kv[0])
    return [t for _, t in tiles], landing_order(world, rank, n_local)


def moe_plan(counts, offsets, row_token, tokens_per_chunk: int, world: int, rank: int,
             N: int, bm: int, bn: int, order: int = ORDER_RANK_OFFSET):
    """Grouped-GEMM tile list for AG-MoE, readiness-sorted.

    Expert e owns output rows offsets[e] .. offsets[e] + counts[e] - 1, whose
    source tokens are row_token[...].  A tile's readiness is the largest
    consume_pos of the chunks holding its tokens; tiles are ordered by
    (readiness, expert, mt, nt) -- least dependent first (talk, "MoE dynamic
    sorting").  With the natural order the key is 0.
    """
    tiles = []
    for e in range(len(counts)):
        me = int(counts[e])
        for mt in range(_ceil_div(me, bm)):
            for nt in range(_ceil_div(N, bn)):
                m0 = int(offsets[e]) + mt * bm
                mr = min(bm, me - mt * bm)
                n0 = nt * bn
                nc = min(bn, N - n0)
                toks = [int(row_token[m0 + i]) for i in range(mr)]
                chunks = sorted({t // tokens_per_chunk for t in toks})
                mask = 0
                for c in chunks:
                    mask |= 1 << c
                key = 0 if order == ORDER_NATURAL else max(consume_pos(c, world, rank) for c in chunks)
                tiles.append(((key, e, mt, nt), (m0, n0, mr, nc, e, mask, key, 0)))
    tiles.sort(key=lambda kv: kv[0])
    return [t for _, t in tiles]
