"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances:
  - index sets: exact, except that a key may be swapped for another only if
    both pooled scores lie within a relative 1e-4 of the oracle's k-th score
    (the kernels' fp32 scores and the oracle's fp64 ones can order such
    near-ties differently);
  - outputs: max-abs 2e-2 for bf16 storage (fp32 accumulation), 1e-4 for fp32,
    5e-3 for fp16 storage. Outputs here stay below ~4 in magnitude, and the
    16-bit rounding of the output and of the probabilities used for P.V each
    contribute at most about 4 * 2^-9 = 7.8e-3 (bf16) or 4 * 2^-11 = 2e-3
    (fp16), together below the bound; fp32 I/O leaves only accumulation-order
    differences.
"""
import numpy as np

NEAR_TIE_REL = 1e-4
TOL = {"bf16": 2e-2, "f32": 1e-4, "f16": 5e-3}


def assert_index_set(gpu, orc, pooled, k, rel=NEAR_TIE_REL, where=""):
    """gpu/orc: int arrays of k indices; pooled: oracle float64 scores of all candidates."""
    gpu = np.asarray(gpu, dtype=np.int64)
    orc = np.asarray(orc, dtype=np.int64)
    assert gpu.shape == (k,), f"{where}: gpu set has shape {gpu.shape}, want ({k},)"
    if k == 0:
        return 0
    assert (gpu >= 0).all() and (gpu < len(pooled)).all(), f"{where}: index out of range"
    assert (np.diff(gpu) > 0).all(), f"{where}: gpu set not strictly ascending"
    tau = pooled[orc].min()
    diff = np.setxor1d(gpu, orc)
    if len(diff):
        dev = np.abs(pooled[diff] - tau)
        bad = diff[dev > rel * tau]
        assert len(bad) == 0, (f"{where}: {len(bad)} keys differ beyond the near-tie band "
                               f"(tau={tau:.6g}, e.g. key {bad[0]} score {pooled[bad[0]]:.6g})")
    return len(diff) // 2


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
