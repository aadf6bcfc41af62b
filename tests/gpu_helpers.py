"""Shared helpers of the GPU tests: input caching, upload, tolerances."""
from __future__ import annotations

import numpy as np

import moe_synth

# Parity bars.
#   Expert outputs, shared outputs, combine and layer output: max relative
#   error 2e-2, rel(a, b) = max|a - b| / max|b| per tensor.
#   Gates and P: a logit rounding difference dl between two fp32 sums moves
#   exp(dl) by ~dl; certified margins assume |dl| << 1e-4, so gates agree to
#   1e-4 relative.  P adds two fp32 summations over T positive terms in
#   different orders, each within (T - 1) 2^-24 relative.
REL_TOL = 2e-2
GATE_TOL = 1e-4


def p_tol(T: int) -> float:
    return GATE_TOL + 2.0 * T * 2.0 ** -24


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def elem_rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float((np.abs(a - b) / np.maximum(np.abs(b), 1e-30)).max())


# Small workloads that span several route blocks (64 tokens) and GEMM tiles
# (128 rows / 64-128 columns / 64-deep K slices) with ragged tails in every
# dimension: T = 300, d = 224 (K tail of 32, column tail of 96), d_ff = 160
# (column tail of 32, K tail of 32).
SMALL = {
    "ragged_bf16": moe_synth.MoEConfig("ragged_bf16", T=300, d=224, N=16, m=1, K=4, K_s=1,
                                       d_ff=160, dtype="bf16"),
    "ragged_f32": moe_synth.MoEConfig("ragged_f32", T=300, d=224, N=16, m=1, K=4, K_s=1,
                                      d_ff=160, dtype="f32"),
    "tiny": moe_synth.CONFIGS["tiny"],
}
FULL = {k: v for k, v in moe_synth.CONFIGS.items() if k != "tiny"}
ALL = dict(SMALL, **FULL)

_cache: dict = {}


def inputs(name: str) -> dict:
    """Seeded inputs of a workload; one workload is kept at a time."""
    if name not in _cache:
        _cache.clear()
        _cache[name] = moe_synth.make_inputs(ALL[name], seed=0)
    return _cache[name]


def sample_tokens(T: int, count: int = 24, seed: int = 11) -> np.ndarray:
    if T <= count:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=count - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), dtype=np.int64)
