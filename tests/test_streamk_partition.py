"""Host logic of the stream-K tail (no GPU): the split of the last tiles into
K pieces and their order, written out here from its contract in
include/tlc.h (TLC_SCHED_STREAMK, tlc_streamk_workspace_bytes), is checked
for the properties the kernel relies on over a sweep of tile counts, grids
and K lengths: every K step of every tail tile is computed exactly once, each
piece has an even number of steps, pieces of one tile are numbered 0..S-1 in
K order and each has its own partial slot, the slots' walk covers every
piece once, and the chosen split beats a round of whole tiles."""
import itertools

import pytest

from tile_level_communication_amd import tlc

MAX_SPLIT = 4
SLOT_BYTES = 256 * 256 * 4
BLOCK_BYTES = 256 + MAX_SPLIT * SLOT_BYTES


def bound(s, KT, S):
    return (s * KT // S) & ~1


def cost(t_sk, G, KT, S):
    per = [0] * G
    for q in range(S * t_sk):
        s = q // t_sk
        per[q % G] += bound(s + 1, KT, S) - bound(s, KT, S)
    return max(per)


def tail(T, G, KT):
    """(sk_from, tiles, split) or None when the schedule stays static."""
    t_dp = T // G * G
    t_sk = T - t_dp
    if t_sk == 0:
        return None
    best, best_cost = 0, KT
    for S in range(2, MAX_SPLIT + 1):
        if 2 * S > KT:
            break
        c = cost(t_sk, G, KT, S) + 2 * (S - 1)
        if c < best_cost:
            best, best_cost = S, c
    return (t_dp, t_sk, best) if best else None


CASES = list(itertools.product([1, 12, 40, 255, 256, 257, 416, 1000],
                               [1, 5, 7, 8, 9, 20, 208, 224, 256],
                               [2, 8, 16, 50, 80]))


@pytest.mark.parametrize("T,G,KT", CASES)
def test_tail_split_properties(T, G, KT):
    cfg = tail(T, G, KT)
    if cfg is None:
        return
    sk_from, t_sk, S = cfg
    assert sk_from % G == 0 and 0 < t_sk < G and sk_from + t_sk == T
    assert 2 <= S <= MAX_SPLIT and t_sk * BLOCK_BYTES <= tlc.streamk_workspace_bytes(G)
    assert cost(t_sk, G, KT, S) < KT
    seen = {}
    # static slots: slot g walks items g, g + G, ...; the tail items follow the
    # whole units, item sk_from + q being piece q // t_sk of tile q % t_sk
    for g in range(G):
        for item in range(g, sk_from + S * t_sk, G):
            if item < sk_from:
                continue
            q = item - sk_from
            s, j = divmod(q, t_sk)
            k0, k1 = bound(s, KT, S), bound(s + 1, KT, S)
            assert 0 <= k0 < k1 <= KT and (k1 - k0) % 2 == 0
            assert (j, s) not in seen
            seen[(j, s)] = (k0, k1)
    assert len(seen) == S * t_sk
    for j in range(t_sk):
        ks = [seen[(j, s)] for s in range(S)]
        assert ks[0][0] == 0 and ks[-1][1] == KT
        assert all(a[1] == b[0] for a, b in zip(ks, ks[1:]))


def test_streamk_workspace_bytes():
    assert tlc.streamk_workspace_bytes(0) == 256 * BLOCK_BYTES
    assert tlc.streamk_workspace_bytes(8) == 8 * BLOCK_BYTES
    assert tlc.streamk_workspace_bytes(-1) == -1


def test_headline_shape_tail():
    """The 8192 x 3200 x 5120 AG-GEMM (416 tiles of 80 K steps): on 256
    workgroups one round of whole tiles, then 160 tiles in three pieces (26,
    26 and 28 steps), at most 54 tail steps per slot; on the 224 a copy-stream
    landing leaves, and on 208 (two even rounds), no tail."""
    assert tail(416, 256, 80) == (256, 160, 3)
    assert cost(160, 256, 80, 3) == 54
    assert tail(416, 224, 80) is None
    assert tail(416, 208, 80) is None
