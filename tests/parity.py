"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerance (floating point): with K the reduction length and max|a|, max|b| the
largest operand magnitudes,
    max |gpu - oracle| <= 2e-3 * sqrt(K) * max|a| * max|b|
    ||gpu - oracle||_F / ||oracle||_F <= 1e-3
The oracle is float64; the GPU accumulates bf16 products in fp32 (MFMA), whose
rounding error grows like sqrt(K) u |a||b| for random signs (u = 2^-24), far
below both bounds; a misplaced row, chunk or tile gives an O(1) relative error
and fails them.  Integer-valued inputs make every fp32 partial sum exact, so
those runs are compared bit for bit.
"""
import sys

import numpy as np

import seeded_inputs as si


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def absmax_bf16(bits) -> float:
    if isinstance(bits, (list, tuple)):
        return max(absmax_bf16(b) for b in bits)
    return float(np.abs(si.bf16_bits_to_f32(bits)).max())


def check_close(got, ref, K, amax, bmax, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in GPU output"
    err = np.abs(got - ref)
    bound = 2e-3 * np.sqrt(K) * amax * bmax
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err.max() <= bound, f"{what}: max err {err.max():.3e} > {bound:.3e}"
    assert rel <= 1e-3, f"{what}: relative Frobenius error {rel:.3e} > 1e-3"
    return float(err.max()), float(rel)


def check_exact(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, f"{what}: {bad[0].size} mismatches, first at {tuple(b[0] for b in bad)}"
