"""Pins for oracle.moe.

* constructed logits whose top-k set is known in closed form;
* all-equal logits (ties): experts 0..k-1, equal gates 1/k;
* k = 2 gates against the closed form 1 / (1 + exp(b - a));
* brute force against numpy's lexsort on small random cases;
* invariants: counts sum to T*k, distinct experts, exclusive-scan offsets,
  expert-local (consume position, token) order, slot/row_token consistency;
* E = 1, k = 1 reduces the grouped GEMM to a dense GEMM; integer inputs exact.
"""
import math

import numpy as np
import pytest

import seeded_inputs as si
from oracle import moe as om
from oracle.gemm import bf16_to_f64


def test_constructed_logits_closed_form():
    T, E, k = 40, 64, 8
    logits = np.zeros((T, E), np.float32)
    for t in range(T):
        for e in range(E):
            logits[t, e] = -float((e * 37 + t) % 64)
    r = om.route(logits, k, 8, 0, 5)
    # (e*37 + t) % 64 == j  <=>  e == (j - t) * 45 mod 64, since 37 * 45 = 1 mod 64
    for t in range(T):
        assert list(r["topk"][t]) == [((j - t) * 45) % 64 for j in range(k)]


def test_ties_go_to_lower_expert():
    logits = np.zeros((6, 16), np.float32)
    r = om.route(logits, 4, 2, 0, 3)
    for t in range(6):
        assert list(r["topk"][t]) == [0, 1, 2, 3]
        np.testing.assert_allclose(r["gates"][t], [0.25] * 4, rtol=0, atol=1e-15)


def test_two_way_gate_closed_form():
    logits = np.array([[0.5, 2.0, -1.0], [3.0, 3.0, 1.0]], np.float32)
    r = om.route(logits, 2, 1, 0, 2)
    assert list(r["topk"][0]) == [1, 0] and list(r["topk"][1]) == [0, 1]
    g = 1.0 / (1.0 + math.exp(float(np.float32(0.5)) - float(np.float32(2.0))))
    assert abs(r["gates"][0, 0] - g) < 1e-15 and abs(r["gates"][0, 1] - (1 - g)) < 1e-15
    assert r["gates"][1, 0] == 0.5


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_vs_lexsort(seed):
    T, E, k = 32, 12, 3
    logits = si.normal_f32((T, E), (990, seed, 0))
    logits[::3, 2] = logits[::3, 5]            # planted ties
    r = om.route(logits, k, 4, seed % 4, 8)
    for t in range(T):
        idx = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        assert list(r["topk"][t]) == list(idx[:k])


@pytest.mark.parametrize("world,rank", [(8, 0), (8, 3), (4, 1)])
def test_routing_invariants(world, rank):
    tpc, E, k = 16, 10, 3
    T = world * tpc
    logits = si.normal_f32((T, E), (991, world, rank))
    r = om.route(logits, k, world, rank, tpc)
    assert int(r["counts"].sum()) == T * k
    assert list(r["offsets"]) == [0] + list(np.cumsum(r["counts"]))
    for t in range(T):
        assert len(set(r["topk"][t])) == k
        assert abs(r["gates"][t].sum() - 1.0) < 1e-12
        assert all(np.diff(r["gates"][t]) <= 0)
    for e in range(E):
        seg = [int(x) for x in r["row_token"][r["offsets"][e]:r["offsets"][e + 1]]]
        members = sorted(t for t in range(T) if e in r["topk"][t])
        assert sorted(seg) == members
        keys = [(((t // tpc) - rank) % world, t) for t in seg]
        assert keys == sorted(keys)
    for t in range(T):
        for j in range(k):
            s = int(r["slot"][t, j])
            e = int(r["topk"][t, j])
            assert r["row_token"][s] == t
            assert r["offsets"][e] <= s < r["offsets"][e + 1]


def test_single_expert_is_dense_gemm():
    world, tpc, H, N = 2, 6, 16, 5
    inp = si.moe_inputs(992, world, tpc, H, N, experts=1, integer=True)
    r = om.route(inp.logits, 1, world, 0, tpc)
    y = om.grouped_gemm(inp.x_chunks, inp.w, r["offsets"], r["row_token"])
    x = np.concatenate([si.bf16_bits_to_f32(c) for c in inp.x_chunks]).astype(np.int64)
    w = si.bf16_bits_to_f32(inp.w[0]).astype(np.int64)
    assert list(r["row_token"]) == list(range(world * tpc))   # rank 0: arrival order = token order
    np.testing.assert_array_equal(y, (x @ w).astype(np.float64))


def test_grouped_gemm_integer_brute_force():
    world, tpc, H, N, E, k = 2, 4, 6, 3, 3, 2
    inp = si.moe_inputs(993, world, tpc, H, N, experts=E, integer=True)
    r = om.route(inp.logits, k, world, 1, tpc)
    y = om.grouped_gemm(inp.x_chunks, inp.w, r["offsets"], r["row_token"])
    x = np.concatenate([si.bf16_bits_to_f32(c) for c in inp.x_chunks]).astype(np.int64)
    for e in range(E):
        w = si.bf16_bits_to_f32(inp.w[e]).astype(np.int64)
        for i in range(r["offsets"][e], r["offsets"][e + 1]):
            t = r["row_token"][i]
            for j in range(N):
                assert y[i, j] == sum(int(x[t, h]) * int(w[h, j]) for h in range(H))
    rows = [0, 5, 15]
    np.testing.assert_array_equal(
        om.grouped_gemm(inp.x_chunks, inp.w, r["offsets"], r["row_token"], rows=rows), y[rows])
