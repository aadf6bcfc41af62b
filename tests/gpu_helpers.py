"""Shared helpers of the GPU tests: input caching, upload, tolerances."""
from __future__ import annotations

import numpy as np

import moe_synth

# Parity bars.
#   Expert outputs, shared outputs, combine and layer output: max relative
#   error 2e-2, rel(a, b) = max|a - b| / max|b| per tensor.
#   Gates: g_i = exp(l_i - max) / Z, so a difference dl in the fp32 logits of
#   the two sides moves g_i by a relative ~2 dl.  Two fp32 dot products of
#   length d summed in different orders differ by about eps sqrt(d) |l|
#   (random-walk rounding, eps = 2^-24); the bound takes eight times that at
#   the largest logit (the same logit error the inputs' top-k margin
#   certificate guards against).  On top come the two sides' exp and division (a few
#   eps) and the sum Z of n positive terms in another order (at most
#   (n - 1) eps relative): (n + 8) eps.  The floor is the 1e-5 the
#   acceptance rules name for gates and P.
#   P: the gate bound plus two fp32 summations over T positive terms in
#   different orders, each within (T - 1) eps relative.
REL_TOL = 2e-2
GATE_TOL = 1e-5
EPS = 2.0 ** -24


def gate_tol(d: int, n: int, max_abs_logit: float) -> float:
    return max(GATE_TOL, 8.0 * EPS * d ** 0.5 * max_abs_logit + (n + 8) * EPS)


def p_tol(T: int, d: int, n: int, max_abs_logit: float) -> float:
    return gate_tol(d, n, max_abs_logit) + 2.0 * T * EPS


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
    # Few rows per expert: the layer and the grouped FFN take the
    # weight-streaming kernels (K tail: d_ff = 160 is 10 k blocks of 16;
    # column tails in both projections).
    "decode_bf16": moe_synth.MoEConfig("decode_bf16", T=40, d=256, N=16, m=2, K=3, K_s=1,
                                       d_ff=160, dtype="bf16"),
    # 256 experts (the most the library takes) and a histogram table of
    # 129 route blocks x 256 experts: too big for the one-pass grouping, so
    # the layer takes the separate scan and scatter kernels.
    "wide_bf16": moe_synth.MoEConfig("wide_bf16", T=2064, d=64, N=64, m=4, K=2, K_s=1,
                                     d_ff=32, dtype="bf16"),
    # Degenerate routings: one kept expert per token; every expert kept
    # (k = n, the order of the slots is the only choice left); and the
    # largest top-k the library takes (k = 64 of n = 128).
    "topk1_bf16": moe_synth.MoEConfig("topk1_bf16", T=130, d=96, N=16, m=1, K=2, K_s=1,
                                      d_ff=64, dtype="bf16"),
    "all_experts_bf16": moe_synth.MoEConfig("all_experts_bf16", T=100, d=96, N=8, m=1, K=8,
                                            K_s=0, d_ff=64, dtype="bf16"),
    "topk64_bf16": moe_synth.MoEConfig("topk64_bf16", T=48, d=64, N=128, m=1, K=64, K_s=0,
                                       d_ff=32, dtype="bf16"),
    # 63 routed experts (the 2B shape's odd count: the last 16-expert group of
    # the small-batch logits holds 15) and a ragged last route block.
    "odd_experts_bf16": moe_synth.MoEConfig("odd_experts_bf16", T=50, d=128, N=63, m=1, K=8,
                                            K_s=1, d_ff=64, dtype="bf16"),
    # One token: a single, mostly empty route block; every group but k is
    # empty and the shared experts see one row.
    "one_token_bf16": moe_synth.MoEConfig("one_token_bf16", T=1, d=64, N=8, m=1, K=3, K_s=1,
                                          d_ff=32, dtype="bf16"),
    # Skewed popularity, no shared experts: some expert gets more than 32
    # rows, so its weights are streamed once per 32 rows.
    "decode_skew_bf16": moe_synth.MoEConfig("decode_skew_bf16", T=64, d=128, N=8, m=1, K=2,
                                            K_s=0, d_ff=96, dtype="bf16", zipf_s=3.0),
}
# The router's edge cases the explainer's "Build it yourself" section lists
# as stretch goals: a single-expert layer (n = 1, so g = 1 for every token),
# with and without a shared expert, on both routers (per-block above 64
# tokens, small-batch at or below) and on the weight-streaming FFN (T = 12);
# and exact ties: centroid row 2j+1 repeats row 2j, so every logit has an
# equal twin on both sides and, with k odd, the k-th choice of every token
# splits a pair: the lower index must win.
SMALL.update({
    "single_expert_bf16": moe_synth.MoEConfig("single_expert_bf16", T=100, d=64, N=1, m=1,
                                              K=1, K_s=0, d_ff=64, dtype="bf16"),
    "single_shared_bf16": moe_synth.MoEConfig("single_shared_bf16", T=40, d=96, N=1, m=1,
                                              K=2, K_s=1, d_ff=64, dtype="bf16"),
    "single_skinny_bf16": moe_synth.MoEConfig("single_skinny_bf16", T=12, d=64, N=1, m=1,
                                              K=1, K_s=0, d_ff=96, dtype="bf16"),
    "single_f32": moe_synth.MoEConfig("single_f32", T=50, d=64, N=1, m=1, K=2, K_s=1,
                                      d_ff=32, dtype="f32"),
    "tie_bf16": moe_synth.MoEConfig("tie_bf16", T=200, d=128, N=16, m=1, K=4, K_s=1,
                                    d_ff=64, dtype="bf16", tie_pairs=True),
    "tie_small_bf16": moe_synth.MoEConfig("tie_small_bf16", T=48, d=128, N=16, m=1, K=4,
                                          K_s=1, d_ff=64, dtype="bf16", tie_pairs=True),
    "tie_wide_bf16": moe_synth.MoEConfig("tie_wide_bf16", T=150, d=2048, N=64, m=1, K=5,
                                         K_s=0, d_ff=32, dtype="bf16", tie_pairs=True),
    "tie_f32": moe_synth.MoEConfig("tie_f32", T=100, d=64, N=8, m=1, K=3, K_s=0, d_ff=32,
                                   dtype="f32", tie_pairs=True, cent_std=0.5),
})
# A flat router: every centroid is zero, so all n logits of every token are
# exactly zero and the tie rule alone picks experts 0 .. k-1 for every token
# (gates 1/n); k of the experts take every token, the rest none.  On both
# routers, the weight-streaming FFN and in fp32.
SMALL.update({
    "flat_bf16": moe_synth.MoEConfig("flat_bf16", T=200, d=128, N=8, m=2, K=2, K_s=1,
                                     d_ff=64, dtype="bf16", flat_router=True),
    "flat_small_bf16": moe_synth.MoEConfig("flat_small_bf16", T=40, d=96, N=8, m=2, K=2,
                                           K_s=1, d_ff=64, dtype="bf16", flat_router=True),
    "flat_f32": moe_synth.MoEConfig("flat_f32", T=50, d=64, N=4, m=2, K=2, K_s=0, d_ff=32,
                                    dtype="f32", flat_router=True),
})
# The granularity sweep at a small size: GShard top-2 of 4 experts (m = 1)
# and the same budget cut eightfold (m = 8: top-16 of 32 experts of width 32).
SMALL.update({
    "gran_m1_bf16": moe_synth.MoEConfig("gran_m1_bf16", T=256, d=128, N=4, m=1, K=2, K_s=0,
                                        d_ff=256, dtype="bf16"),
    "gran_m8_bf16": moe_synth.MoEConfig("gran_m8_bf16", T=256, d=128, N=4, m=8, K=2, K_s=0,
                                        d_ff=32, dtype="bf16"),
})
FULL = {k: v for k, v in moe_synth.CONFIGS.items() if k != "tiny"}
FULL.update(moe_synth.GRANULARITY)
# Tile lists that span more than one round of the GEMM launches' 512
# workgroup slots (so the tail-claiming path runs) on small matrices, with
# an odd number of K slices in the up projection (d = 416: 13 slices of 32)
# and column tails in both projections.
FULL["multi_round_bf16"] = moe_synth.MoEConfig("multi_round_bf16", T=4096, d=416, N=16, m=1,
                                               K=9, K_s=1, d_ff=256, dtype="bf16")
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
