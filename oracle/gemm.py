"""Oracle for AllGather-GEMM and GEMM-ReduceScatter (test infrastructure only).

Plain definitions in float64; the swizzled, overlapped method reaches the same
values up to rounding order because it only reorders tiles and transfers
(AutoOverlap §6.2/§7.2: the tile-order knobs keep semantics unchanged; DITRON
paper notes, the §4.3 text on training deployment: adapted kernels are
bitwise equal to the native ones).

* AllGather-GEMM (DITRON §2 and §4.1, AG-GEMM workload; talk, swizzling
  section): every rank r holds one row chunk A_r of the activations; after the
  all-gather each rank computes C = concat(A_0, ..., A_{W-1}) @ B with its own
  weight shard B.  Chunks are concatenated in rank order, whatever order they
  arrive in.
* GEMM-ReduceScatter (DITRON §4.1, GEMM-RS workload; talk, GEMM-ReduceScatter
  example with per-tile notify and a separate reduce kernel): every rank s
  computes a full partial product P_s = A_s @ B_s over its K shard; rank r owns
  rows [r*R, (r+1)*R) of the sum, out_r = sum_s P_s[rows of r].  The sum is taken
  in ascending s (the reading that makes the result independent of arrival
  order).  On one GPU only the local partial P_r is computed; the other ranks'
  slices for rank r arrive as inputs ("remote partials").

* GEMM-AllReduce (DITRON §4, the tensor-parallel kernels GEMM-AllReduce next
  to AG-GEMM and GEMM-RS; §5.1 reports it separately): every rank ends with the
  whole sum C = sum_s P_s.  Taken here as the reduce-scatter above followed by
  an all-gather of the reduced slices: rows of chunk r are rank r's own reduce,
  rows of chunk c != r are the slice rank c reduced ("gathered" inputs on one
  GPU).

Inputs are bf16 bit patterns (uint16) and fp32 arrays from ``seeded_inputs``;
bf16 -> float64 widening is exact.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns: the bf16 value is the top half of an fp32."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def gather_rows(a_chunks):
    """concat_c A_c in rank order (the all-gather's result), as float64."""
    return np.concatenate([bf16_to_f64(a) for a in a_chunks], axis=0)


def ag_gemm(a_chunks, b_kn) -> np.ndarray:
    """C = concat(A_0..A_{W-1}) @ B, float64.  b_kn is the logical K x N weight."""
    return gather_rows(a_chunks) @ bf16_to_f64(b_kn)


def ag_gemm_rows(a_chunks, b_kn, rows) -> np.ndarray:
    """Selected rows of C (global row indices), for sampled checks at full size."""
    rows = np.asarray(rows, dtype=np.int64)
    R = a_chunks[0].shape[0]
    a = np.stack([bf16_to_f64(a_chunks[int(i) // R][int(i) % R]) for i in rows])
    return a @ bf16_to_f64(b_kn)


def gemm_partial(a_local, b_kn, rows=None) -> np.ndarray:
    """Local partial product P = A_local @ B (float64); optionally only some rows."""
    a = a_local if rows is None else a_local[np.asarray(rows, dtype=np.int64)]
    return bf16_to_f64(a) @ bf16_to_f64(b_kn)


def reduce_slice(local_slice: np.ndarray, remote: dict, world: int, rank: int) -> np.ndarray:
    """out_r = sum over s = 0..W-1 in ascending order of S_s, with S_r the local slice
    and S_s (s != r) the partial that rank s computed for rank r's rows."""
    out = np.zeros_like(local_slice, dtype=np.float64)
    for s in range(world):
        term = local_slice if s == rank else np.asarray(remote[s], dtype=np.float64)
        out = out + term
    return out


def gemm_rs(a_local, b_kn, remote: dict, world: int, rank: int):
    """(P, out): the full local partial (M x N) and rank's reduced slice (R x N)."""
    p = gemm_partial(a_local, b_kn)
    R = p.shape[0] // world
    out = reduce_slice(p[rank * R:(rank + 1) * R], remote, world, rank)
    return p, out


def gemm_rs_rows(a_local, b_kn, remote: dict, world: int, rank: int, local_rows):
    """Sampled version: rows are indices inside rank's slice (0..R-1).  Returns
    (P rows of the slice, out rows)."""
    R = a_local.shape[0] // world
    local_rows = np.asarray(local_rows, dtype=np.int64)
    p = gemm_partial(a_local, b_kn, rank * R + local_rows)
    sub = {s: np.asarray(v)[local_rows] for s, v in remote.items()}
    return p, reduce_slice(p, sub, world, rank)


def gemm_ar(a_local, b_kn, remote: dict, gathered: dict, world: int, rank: int):
    """(P, C): the local partial (M x N) and the all-reduced product C (M x N),
    whose row chunk `rank` is this rank's reduced slice and whose row chunk c
    (c != rank) is gathered[c], the slice rank c reduced."""
    p, out = gemm_rs(a_local, b_kn, remote, world, rank)
    R = p.shape[0] // world
    c = np.empty_like(p)
    for ch in range(world):
        c[ch * R:(ch + 1) * R] = out if ch == rank else np.asarray(gathered[ch], dtype=np.float64)
    return p, c


def blocked_gemm_f32(a_rows, b_kn, units):
    """The blocked fp32 GEMM: C (fp32) assembled tile by tile in the given unit
    order (m0, n0, m_rows, n_cols, ...), each tile accumulating its products in
    fp32 over k = 0, 1, ..., K-1 in increasing order (DITRON §3.1, core-level
    tiles; the tile order is the only thing the swizzle changes).  a_rows: M x K
    bf16 bits (the gathered rows), b_kn: K x N bf16 bits.  Slow (one fp32
    rank-1 update per k): for small shapes only."""
    a = bf16_to_f64(a_rows).astype(np.float32)
    b = bf16_to_f64(b_kn).astype(np.float32)
    M, K = a.shape
    N = b.shape[1]
    c = np.full((M, N), np.nan, dtype=np.float32)
    for u in units:
        m0, n0, mr, nc = u[0], u[1], u[2], u[3]
        acc = np.zeros((mr, nc), dtype=np.float32)
        for k in range(K):
            acc += a[m0:m0 + mr, k:k + 1] * b[k:k + 1, n0:n0 + nc]
        c[m0:m0 + mr, n0:n0 + nc] = acc
    return c
