"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module only draws numbers: it holds none of the method's arithmetic (no
GEMM, no reduction, no routing, no tile ordering).  Both the oracle under
``oracle/`` and the HIP path read the arrays it returns, so the two sides see
bit-identical inputs without sharing any compute code.

Recipe
------
* Generator: numpy ``PCG64`` seeded with ``SeedSequence([0, workload, tensor, chunk])``.
* Floating-point draws: ``standard_normal(dtype=float32)``, multiplied by the
  stated standard deviation in fp32, then rounded to bfloat16 with
  round-to-nearest-even.  bf16 tensors are returned as their raw ``uint16`` bit
  patterns; fp32 tensors (router logits, remote partial sums) stay fp32.
* Integer-valued draws (used for bit-exact tests): uniform integers in
  ``[-4, 4]`` stored as bf16 bit patterns; every such value and every partial
  sum of products with ``K * 16 < 2**24`` is exact in fp32.

Workloads (tensor shapes are the ones the AG-GEMM / GEMM-RS / AG-MoE workloads
of the tile-level communication pages use; see ``WORKLOADS``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# tensor ids inside a seed tuple
T_A = 0        # activations: A chunks (AG), local A (RS), tokens X (MoE)
T_B = 1        # weights: B (AG/RS), stacked expert weights (MoE)
T_REMOTE = 2   # fp32 partial sums of the emulated peer ranks (RS)
T_LOGITS = 3   # fp32 router logits (MoE)
T_GATHERED = 4  # fp32 reduced slices of the emulated peer ranks (GEMM-AllReduce)


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 generator for the seed tuple ``(0, *key)``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, *[int(k) for k in key]])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(shape, key, std: float = 1.0) -> np.ndarray:
    g = rng_for(*key)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_bf16(shape, key, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16; uint16 bit patterns."""
    return f32_to_bf16_bits(normal_f32(shape, key, std))


def int_bf16(shape, key, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 bit patterns (exact)."""
    g = rng_for(*key)
    v = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


def int_f32(shape, key, lo: int = -4, hi: int = 4) -> np.ndarray:
    g = rng_for(*key)
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "ag", "rs" or "moe"
    world: int                # number of chunks W
    rows_per_chunk: int       # R (tokens per chunk for MoE)
    n: int
    k: int
    a_std: float = 1.0
    b_std: float = 1.0
    remote_std: float = 0.0   # RS only
    experts: int = 0          # MoE only
    topk: int = 0             # MoE only
    tile: tuple = (256, 256)  # default BM x BN
    note: str = ""

    @property
    def m(self) -> int:
        return self.world * self.rows_per_chunk


WORKLOADS = {
    # AllGather-GEMM, tiny: 2 chunks of 128x512, B 512x256.
    0: Workload("ag_tiny_w2_256x256x512", "ag", 2, 128, 256, 512, tile=(128, 128)),
    # GEMM-ReduceScatter: A 4096x2048 (K shard), B 2048x4096, both N(0,1)/sqrt(K).
    1: Workload("rs_w4_4096x4096x2048", "rs", 4, 1024, 4096, 2048,
                a_std=1.0 / math.sqrt(2048), b_std=1.0 / math.sqrt(2048),
                remote_std=1.0 / math.sqrt(2048)),
    # AllGather-GEMM, Qwen3-32B-like FFN up: 8 chunks of 1024x5120, B 5120x3200.
    2: Workload("ag_qwen3_32b_ffn_up_w8_8192x3200x5120", "ag", 8, 1024, 3200, 5120,
                a_std=1.0, b_std=0.02),
    # GEMM-ReduceScatter, long-context FFN down: A 131072x3200, B 3200x5120.
    3: Workload("rs_ffn_down_128k_w8_131072x5120x3200", "rs", 8, 16384, 5120, 3200,
                a_std=1.0, b_std=0.02, remote_std=0.02 * math.sqrt(3200)),
    # AG-MoE: 8 chunks of 512 tokens x 2048 hidden, 64 experts, top-8, expert W 2048x768.
    4: Workload("ag_moe_w8_t4096_e64_top8_h2048_n768", "moe", 8, 512, 768, 2048,
                a_std=1.0, b_std=0.02, experts=64, topk=8),
}


@dataclass
class AGInputs:
    a_chunks: list            # W arrays, each R x K bf16 bits
    b: np.ndarray             # K x N bf16 bits (logical layout)


@dataclass
class RSInputs:
    a: np.ndarray             # M x K bf16 bits (local K shard)
    b: np.ndarray             # K x N bf16 bits
    remote: dict              # s -> R x N fp32, for every s != rank


@dataclass
class ARInputs:
    a: np.ndarray             # M x K bf16 bits (local K shard)
    b: np.ndarray             # K x N bf16 bits
    remote: dict              # s -> R x N fp32, for every s != rank (partials for rank's rows)
    gathered: dict            # c -> R x N fp32, for every c != rank (rank c's reduced slice)


@dataclass
class MoEInputs:
    x_chunks: list            # W arrays, each Tc x H bf16 bits
    logits: np.ndarray        # T x E fp32
    w: np.ndarray             # E x H x N bf16 bits (per-expert K x N)


def ag_inputs(wl_id: int, world: int, rows: int, n: int, k: int, a_std=1.0, b_std=1.0,
              integer: bool = False) -> AGInputs:
    if integer:
        a = [int_bf16((rows, k), (wl_id, T_A, c)) for c in range(world)]
        b = int_bf16((k, n), (wl_id, T_B, 0))
    else:
        a = [normal_bf16((rows, k), (wl_id, T_A, c), a_std) for c in range(world)]
        b = normal_bf16((k, n), (wl_id, T_B, 0), b_std)
    return AGInputs(a, b)


def rs_inputs(wl_id: int, world: int, rank: int, rows: int, n: int, k: int, a_std=1.0,
              b_std=1.0, remote_std=1.0, integer: bool = False, remote_zero: bool = False) -> RSInputs:
    m = world * rows
    if integer:
        a = np.concatenate([int_bf16((rows, k), (wl_id, T_A, c)) for c in range(world)])
        b = int_bf16((k, n), (wl_id, T_B, 0))
        remote = {s: int_f32((rows, n), (wl_id, T_REMOTE, s), -64, 64) for s in range(world) if s != rank}
    else:
        a = np.concatenate([normal_bf16((rows, k), (wl_id, T_A, c), a_std) for c in range(world)])
        b = normal_bf16((k, n), (wl_id, T_B, 0), b_std)
        remote = {s: normal_f32((rows, n), (wl_id, T_REMOTE, s), remote_std)
                  for s in range(world) if s != rank}
    if remote_zero:
        remote = {s: np.zeros((rows, n), np.float32) for s in remote}
    assert a.shape == (m, k)
    return RSInputs(a, b, remote)


def ar_inputs(wl_id: int, world: int, rank: int, rows: int, n: int, k: int, a_std=1.0,
              b_std=1.0, remote_std=1.0, integer: bool = False) -> ARInputs:
    """GEMM-RS inputs plus the reduced slices the other ranks produce: each is a
    sum of `world` partials, so it is drawn with std remote_std * sqrt(world)
    (integer case: uniform integers in [-256, 256])."""
    rs = rs_inputs(wl_id, world, rank, rows, n, k, a_std, b_std, remote_std, integer)
    if integer:
        gathered = {c: int_f32((rows, n), (wl_id, T_GATHERED, c), -256, 256)
                    for c in range(world) if c != rank}
    else:
        gathered = {c: normal_f32((rows, n), (wl_id, T_GATHERED, c), remote_std * math.sqrt(world))
                    for c in range(world) if c != rank}
    return ARInputs(rs.a, rs.b, rs.remote, gathered)


def moe_inputs(wl_id: int, world: int, tokens: int, hidden: int, n: int, experts: int,
               a_std=1.0, b_std=0.02, integer: bool = False) -> MoEInputs:
    if integer:
        x = [int_bf16((tokens, hidden), (wl_id, T_A, c)) for c in range(world)]
        w = int_bf16((experts, hidden, n), (wl_id, T_B, 0))
    else:
        x = [normal_bf16((tokens, hidden), (wl_id, T_A, c), a_std) for c in range(world)]
        w = normal_bf16((experts, hidden, n), (wl_id, T_B, 0), b_std)
    logits = normal_f32((world * tokens, experts), (wl_id, T_LOGITS, 0), 1.0)
    return MoEInputs(x, logits, w)


def workload_inputs(wl_id: int, rank: int = 0, integer: bool = False):
    wl = WORKLOADS[wl_id]
    if wl.kind == "ag":
        return ag_inputs(wl_id, wl.world, wl.rows_per_chunk, wl.n, wl.k, wl.a_std, wl.b_std, integer)
    if wl.kind == "rs":
        return rs_inputs(wl_id, wl.world, rank, wl.rows_per_chunk, wl.n, wl.k, wl.a_std, wl.b_std,
                         wl.remote_std, integer)
    return moe_inputs(wl_id, wl.world, wl.rows_per_chunk, wl.k, wl.n, wl.experts, wl.a_std,
                      wl.b_std, integer)
