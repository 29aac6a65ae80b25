"""Pins for oracle.gemm: checks that do not reuse the oracle's own formulas.

* exact rational arithmetic (fractions.Fraction) on tiny shapes, with the
  classical bound |fl(sum) - sum| <= gamma_K * sum |a||b| for float64 dot
  products (gamma_K = K u / (1 - K u), u = 2^-53);
* integer-valued inputs, for which every float64 (and fp32) sum is exact, so the
  oracle must equal Python integer arithmetic bit for bit -- a wrong chunk
  order, a transposed operand or an off-by-one row fails exactly;
* special cases: one chunk is a plain GEMM (torch.matmul in float64); all
  remote partials zero gives the local slice back; a constructed sum whose value
  depends on the summation order pins the ascending-rank order of the reduce.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import gemm as og


def _exact(a_bits, b_bits):
    a = si.bf16_bits_to_f32(a_bits).astype(np.float64)
    b = si.bf16_bits_to_f32(b_bits).astype(np.float64)
    M, K = a.shape
    N = b.shape[1]
    c = [[sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(K))
          for j in range(N)] for i in range(M)]
    absum = [[sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j]))) for k in range(K))
              for j in range(N)] for i in range(M)]
    return c, absum


@pytest.mark.parametrize("world,rows,k,n", [(3, 5, 7, 4), (2, 4, 16, 3), (1, 6, 9, 5)])
def test_ag_gemm_vs_exact_rational(world, rows, k, n):
    inp = si.ag_inputs(901, world, rows, n, k, a_std=1.0, b_std=0.5)
    c = og.ag_gemm(inp.a_chunks, inp.b)
    a_all = np.concatenate(inp.a_chunks)
    exact, absum = _exact(a_all, inp.b)
    u = 2.0 ** -53
    gamma = k * u / (1 - k * u)
    for i in range(world * rows):
        for j in range(n):
            err = abs(Fraction(float(c[i, j])) - exact[i][j])
            assert err <= Fraction(gamma) * absum[i][j] + Fraction(1, 2 ** 1074)


@pytest.mark.parametrize("world,rows,k,n", [(4, 3, 20, 5), (8, 2, 33, 7)])
def test_ag_gemm_integer_exact_per_chunk(world, rows, k, n):
    inp = si.ag_inputs(902, world, rows, n, k, integer=True)
    c = og.ag_gemm(inp.a_chunks, inp.b)
    b = si.bf16_bits_to_f32(inp.b).astype(np.int64)
    for ch in range(world):
        a = si.bf16_bits_to_f32(inp.a_chunks[ch]).astype(np.int64)
        for i in range(rows):
            for j in range(n):
                want = sum(int(a[i, kk]) * int(b[kk, j]) for kk in range(k))
                assert c[ch * rows + i, j] == want


def test_ag_gemm_rows_matches_full():
    inp = si.ag_inputs(903, 4, 16, 24, 40)
    full = og.ag_gemm(inp.a_chunks, inp.b)
    rows = [0, 15, 16, 33, 63]
    np.testing.assert_array_equal(og.ag_gemm_rows(inp.a_chunks, inp.b, rows), full[rows])


def test_single_chunk_is_plain_gemm():
    inp = si.ag_inputs(904, 1, 40, 24, 56)
    c = og.ag_gemm(inp.a_chunks, inp.b)
    a = torch.from_numpy(si.bf16_bits_to_f32(inp.a_chunks[0])).double()
    b = torch.from_numpy(si.bf16_bits_to_f32(inp.b)).double()
    ref = torch.matmul(a, b).numpy()
    np.testing.assert_allclose(c, ref, rtol=1e-13, atol=1e-13)


def test_bf16_widening_known_values():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x4049 = 3.140625, 0x0000 = 0
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x4049, 0x0000], np.uint16)
    np.testing.assert_array_equal(og.bf16_to_f64(bits), [1.0, -2.0, 0.25, 3.140625, 0.0])


@pytest.mark.parametrize("world,rank", [(4, 0), (4, 3), (3, 1)])
def test_gemm_rs_integer_exact(world, rank):
    rows, k, n = 3, 10, 4
    inp = si.rs_inputs(905, world, rank, rows, n, k, integer=True)
    p, out = og.gemm_rs(inp.a, inp.b, inp.remote, world, rank)
    a = si.bf16_bits_to_f32(inp.a).astype(np.int64)
    b = si.bf16_bits_to_f32(inp.b).astype(np.int64)
    for i in range(world * rows):
        for j in range(n):
            assert p[i, j] == sum(int(a[i, kk]) * int(b[kk, j]) for kk in range(k))
    for i in range(rows):
        for j in range(n):
            want = 0
            for s in range(world):
                if s == rank:
                    want += sum(int(a[rank * rows + i, kk]) * int(b[kk, j]) for kk in range(k))
                else:
                    want += int(inp.remote[s][i, j])
            assert out[i, j] == want


def test_gemm_rs_zero_remote_gives_local_slice():
    world, rank, rows = 4, 2, 8
    inp = si.rs_inputs(906, world, rank, rows, 12, 32, remote_zero=True)
    p, out = og.gemm_rs(inp.a, inp.b, inp.remote, world, rank)
    np.testing.assert_array_equal(out, p[rank * rows:(rank + 1) * rows])


def test_reduce_order_is_ascending_rank():
    # S_0 = 2^53, S_1 = 1, S_2 = -2^53 (local, rank 2).  Ascending order gives
    # (2^53 + 1) -> 2^53 (ties to even), then 0.  Any order that adds the 1 last
    # gives 1; descending order gives (-2^53 + 1) + 2^53 = 1.
    local = np.array([[-2.0 ** 53]])
    remote = {0: np.array([[2.0 ** 53]]), 1: np.array([[1.0]])}
    out = og.reduce_slice(local, remote, 3, 2)
    assert out[0, 0] == 0.0


def test_gemm_rs_rows_matches_full():
    world, rank, rows = 4, 1, 16
    inp = si.rs_inputs(907, world, rank, rows, 20, 24, remote_std=0.3)
    p, out = og.gemm_rs(inp.a, inp.b, inp.remote, world, rank)
    sel = [0, 7, 15]
    ps, outs = og.gemm_rs_rows(inp.a, inp.b, inp.remote, world, rank, sel)
    np.testing.assert_array_equal(ps, p[rank * rows + np.array(sel)])
    np.testing.assert_array_equal(outs, out[sel])


@pytest.mark.parametrize("world,rank", [(4, 1), (3, 2), (2, 0)])
def test_gemm_ar_integer_exact(world, rank):
    rows, k, n = 3, 8, 5
    inp = si.ar_inputs(908, world, rank, rows, n, k, integer=True)
    p, c = og.gemm_ar(inp.a, inp.b, inp.remote, inp.gathered, world, rank)
    a = si.bf16_bits_to_f32(inp.a).astype(np.int64)
    b = si.bf16_bits_to_f32(inp.b).astype(np.int64)
    for ch in range(world):
        for i in range(rows):
            for j in range(n):
                if ch != rank:
                    assert c[ch * rows + i, j] == inp.gathered[ch][i, j]
                    continue
                want = sum(int(inp.remote[s][i, j]) for s in range(world) if s != rank)
                want += sum(int(a[rank * rows + i, kk]) * int(b[kk, j]) for kk in range(k))
                assert c[ch * rows + i, j] == want


def test_gemm_ar_consistent_shards_give_unsharded_product():
    """W ranks each hold a K shard (A_s, B_s).  With every peer input built
    from those shards by brute force, every rank's all-reduced C is the
    unsharded product [A_0 .. A_{W-1}] @ [B_0; ..; B_{W-1}] (K concatenated),
    computed here by one integer matrix product."""
    world, rows, n, ks = 3, 4, 6, 5
    M = world * rows
    shards = [si.rs_inputs(909 + s, world, 0, rows, n, ks, integer=True) for s in range(world)]
    A = [si.bf16_bits_to_f32(sh.a).astype(np.int64) for sh in shards]
    B = [si.bf16_bits_to_f32(sh.b).astype(np.int64) for sh in shards]

    def partial(s, i, j):  # brute force P_s[i, j]
        return sum(int(A[s][i, kk]) * int(B[s][kk, j]) for kk in range(ks))

    full = np.concatenate(A, axis=1) @ np.concatenate(B, axis=0)
    for rank in range(world):
        remote = {s: np.array([[partial(s, rank * rows + i, j) for j in range(n)] for i in range(rows)],
                              np.float32) for s in range(world) if s != rank}
        gathered = {c: np.array([[sum(partial(s, c * rows + i, j) for s in range(world))
                                  for j in range(n)] for i in range(rows)], np.float32)
                    for c in range(world) if c != rank}
        _, c = og.gemm_ar(shards[rank].a, shards[rank].b, remote, gathered, world, rank)
        assert c.shape == (M, n)
        np.testing.assert_array_equal(c, full.astype(np.float64))


def test_blocked_f32_tile_order_never_changes_the_result():
    """The blocked fp32 GEMM gives the same bits in every tile order -- the
    communication-aware orders of every rank, the natural order, reversed and
    shuffled orders -- covers C exactly once, and stays within the stated
    tolerance of the float64 definition."""
    from oracle import plan as op
    W, R, K, N = 3, 40, 48, 56
    inp = si.ag_inputs(911, W, R, N, K)
    a_rows = np.concatenate(inp.a_chunks)
    ref64 = og.ag_gemm(inp.a_chunks, inp.b)
    base, _ = op.chunk_plan(op.AG, W, 0, W * R, N, R, 32, 32, op.ORDER_NATURAL, 1)
    first = og.blocked_gemm_f32(a_rows, inp.b, base)
    assert not np.isnan(first).any()
    rng = np.random.default_rng(5)
    orders = [list(reversed(base)), [base[i] for i in rng.permutation(len(base))]]
    for rank in range(W):
        for mode in (op.AG, op.RS):
            orders.append(op.chunk_plan(mode, W, rank, W * R, N, R, 32, 32, op.ORDER_RANK_OFFSET, 2)[0])
    for units in orders:
        got = og.blocked_gemm_f32(a_rows, inp.b, units)
        assert np.array_equal(got.view(np.uint32), first.view(np.uint32))
    amax = float(np.abs(si.bf16_bits_to_f32(a_rows)).max())
    bmax = float(np.abs(si.bf16_bits_to_f32(inp.b)).max())
    err = np.abs(first.astype(np.float64) - ref64)
    assert err.max() <= 2e-3 * np.sqrt(K) * amax * bmax
    assert np.linalg.norm(first - ref64) / np.linalg.norm(ref64) <= 1e-3


def test_blocked_f32_integer_inputs_exact():
    """Integer-valued inputs make every fp32 partial sum exact: the blocked
    fp32 GEMM then equals the integer brute force."""
    from oracle import plan as op
    W, R, K, N = 2, 9, 12, 10
    inp = si.ag_inputs(912, W, R, N, K, integer=True)
    a_rows = np.concatenate(inp.a_chunks)
    units, _ = op.chunk_plan(op.AG, W, 1, W * R, N, R, 8, 8, op.ORDER_RANK_OFFSET, 1)
    got = og.blocked_gemm_f32(a_rows, inp.b, units)
    a = si.bf16_bits_to_f32(a_rows).astype(np.int64)
    b = si.bf16_bits_to_f32(inp.b).astype(np.int64)
    for i in range(W * R):
        for j in range(N):
            assert got[i, j] == sum(int(a[i, k]) * int(b[k, j]) for k in range(K))
