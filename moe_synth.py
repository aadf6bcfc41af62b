"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It only draws random numbers and rounds them to the storage type; it computes
nothing the layer computes, with one exception that is a property of the
inputs, not an output: the top-k margin certificate (fp64 logits of the stored
values) used to redraw tokens whose routing decision would sit within 1e-4 of a
tie.

Workload shapes follow the DeepSeekMoE pages: fine-grained segmentation gives
n = m*N routed experts of which k = m*K - K_s are kept per token, plus K_s
always-on shared experts (deepforge.srivtx.xyz "DeepSeekMoE", sections
"Routing in a classic MoE layer" and "What the 16B configuration looks like").
The 16B shape (64 routed, 2 shared, 6 routed active, d = 2048) and the 145B
shape (128 routed, 4 shared, 12 active) come from the latter section; T, d_ff
and the value distributions are this project's synthetic stand-ins.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Stream ids: one independent PCG64 stream per tensor.
_STREAM = {"u": 1, "centroids": 2, "w1": 3, "w3": 4, "w2": 5,
           "ws1": 6, "ws3": 7, "ws2": 8, "redraw": 9, "dh": 10}

MARGIN = 1e-4
EPS32 = 2.0 ** -24  # unit roundoff of fp32


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    N: int
    m: int
    K: int
    K_s: int
    d_ff: int
    dtype: str
    cent_std: float | None = None   # None: 1/sqrt(d)
    w_std: float = 0.02
    zipf_s: float | None = None     # Zipf exponent on centroid row norms
    tie_pairs: bool = False         # centroid row 2j+1 repeats row 2j: exact logit ties
    flat_router: bool = False       # every centroid zero: all n logits tie at zero

    @property
    def n(self) -> int:
        return self.m * self.N

    @property
    def k(self) -> int:
        return self.m * self.K - self.K_s

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  (N, m, K) factorisations: only m*N and m*K - K_s enter the
# layer; 16B is (16, 4, 2) as on the pages (64 routed = 16 x 4, 8 = 2 x 4 active
# incl. 2 shared); 2B-shaped is 63 routed + 1 shared with 7 routed kept; the 145B
# granularity is not printed, m = 4 is used.
CONFIGS = {
    "tiny": MoEConfig("tiny", T=64, d=64, N=4, m=4, K=1, K_s=1, d_ff=32,
                      dtype=F32, cent_std=0.02),
    "2b": MoEConfig("2b", T=8192, d=1280, N=63, m=1, K=8, K_s=1, d_ff=896,
                    dtype=BF16),
    "16b": MoEConfig("16b", T=4096, d=2048, N=16, m=4, K=2, K_s=2, d_ff=1408,
                     dtype=BF16),
    "145b": MoEConfig("145b", T=4096, d=4096, N=32, m=4, K=4, K_s=4, d_ff=1408,
                      dtype=BF16, zipf_s=1.1),
    "16b_decode": MoEConfig("16b_decode", T=64, d=2048, N=16, m=4, K=2, K_s=2,
                            d_ff=1408, dtype=BF16),
}


# Granularity sweep at a fixed budget: the 16B shape's N = 16 experts of width
# D = 4 x 1408 = 5632, K = 2 of them active, cut into m finer experts each
# (n = 16m experts of width D/m, k = 2m kept) with no shared experts, so the
# total and the activated expert parameters stay the same for every m; m = 1
# is GShard's top-2 layer (DeepSeekMoE explainer, "Routing in a classic MoE
# layer" and the fine-grained segmentation it describes).
GRANULARITY = {
    f"gran_m{m}": MoEConfig(f"gran_m{m}", T=4096, d=2048, N=16, m=m, K=2, K_s=0,
                            d_ff=5632 // m, dtype=BF16)
    for m in (1, 2, 4, 8)
}


def _rng(seed: int, stream: str, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, _STREAM[stream], sub])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Stored values as fp32 (exact for both storage types)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def zipf_row_scale(n: int, s: float) -> np.ndarray:
    """r_i = i^-s / mean_j j^-s for i = 1..n (mean one)."""
    r = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return r / r.mean()


def _weights(rng: np.random.Generator, groups: int, rows: int, cols: int,
             std: float, dtype: str) -> np.ndarray:
    """[groups][rows][cols], drawn group by group to cap host memory."""
    out = np.empty((groups, rows, cols), np.uint16 if dtype == BF16 else np.float32)
    for g in range(groups):
        out[g] = _store(_normal(rng, (rows, cols), std), dtype)
    return out


def certified_margin(d: int, max_abs_logit: float) -> float:
    """Smallest top-k gap the inputs must keep: 1e-4, or eight times the
    typical difference between two fp32 summation orders of a length-d dot
    product near the largest logit (random-walk rounding, eps sqrt(d) |l|),
    whichever is larger.  bf16 products are exact in fp32, so only the order
    of the sums differs between two correct fp32 implementations."""
    return max(MARGIN, 8.0 * EPS32 * math.sqrt(d) * max_abs_logit)


def twin_groups(c32: np.ndarray) -> np.ndarray:
    """Group id per centroid row: equal rows (bit for bit) share an id."""
    _, gid = np.unique(np.ascontiguousarray(c32).view(np.uint32), axis=0, return_inverse=True)
    return np.asarray(gid).reshape(-1)


def margin_violations(u32: np.ndarray, c32: np.ndarray, k: int,
                      margin: float = MARGIN) -> np.ndarray:
    """Tokens whose top-(k+1) fp64 logits have an adjacent gap <= margin.

    Returns a boolean mask over tokens.  With k = n only the order gaps inside
    the top k are checked.  Experts with identical centroid rows tie exactly in
    any summation order (the tie rule decides between them), so a gap between
    two such experts is not a violation.
    """
    n = c32.shape[0]
    lg = u32.astype(np.float64) @ c32.astype(np.float64).T
    top = min(k + 1, n)
    if top < 2:
        return np.zeros(u32.shape[0], dtype=bool)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :top]
    part = np.take_along_axis(lg, order, axis=1)
    gaps = part[:, :-1] - part[:, 1:]
    g = twin_groups(c32)[order]
    twin = g[:, :-1] == g[:, 1:]
    return ((gaps <= margin) & ~twin).any(axis=1)


def max_abs_logit(u32: np.ndarray, c32: np.ndarray) -> float:
    return float(np.abs(u32.astype(np.float64) @ c32.astype(np.float64).T).max())


def make_router_inputs(cfg: MoEConfig, seed: int = 0, certify: bool = True):
    """u [T,d] and centroids [n,d] in storage type, plus the redraw count.

    With certify, every token's top-(k+1) logits keep adjacent gaps above
    certified_margin (tokens that do not are redrawn from their own stream)."""
    T, d, n = cfg.T, cfg.d, cfg.n
    u = _store(_normal(_rng(seed, "u"), (T, d), 1.0), cfg.dtype)
    cstd = cfg.cent_std if cfg.cent_std is not None else 1.0 / math.sqrt(d)
    c = _normal(_rng(seed, "centroids"), (n, d), cstd)
    if cfg.zipf_s is not None:
        c *= zipf_row_scale(n, cfg.zipf_s).astype(np.float32)[:, None]
    if cfg.tie_pairs:
        c[1::2] = c[0:n - 1:2]
    if cfg.flat_router:
        c = np.zeros((n, d), np.float32)  # +0 everywhere: one twin group
    cent = _store(c, cfg.dtype)
    redraws = 0
    if certify:
        c32 = as_f32(cent)
        rr = _rng(seed, "redraw")
        rounds = 0
        while True:
            margin = certified_margin(d, max_abs_logit(as_f32(u), c32))
            bad = margin_violations(as_f32(u), c32, cfg.k, margin)
            if not bad.any():
                break
            while bad.any():
                idx = np.nonzero(bad)[0]
                redraws += idx.size
                u[idx] = _store(_normal(rr, (idx.size, d), 1.0), cfg.dtype)
                sub = margin_violations(as_f32(u[idx]), c32, cfg.k, margin)
                bad = np.zeros(T, dtype=bool)
                bad[idx[sub]] = True
                rounds += 1
                if rounds > 1000:
                    raise RuntimeError("margin certification did not converge")
    return u, cent, redraws


# Balance-loss coefficient alpha_1 the explainer gives (section "Expert-level
# balance loss"): 0.01 for the 2B runs, 0.001 at 16B.
BALANCE_ALPHA = {"2b": 0.01, "16b": 0.001}


def make_upstream_grad(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Gradient of a loss with respect to the layer output h [T][d] for the
    backward pass: standard normals in the workload's storage type."""
    return _store(_normal(_rng(seed, "dh"), (cfg.T, cfg.d), 1.0), cfg.dtype)


def make_inputs(cfg: MoEConfig, seed: int = 0, certify: bool = True) -> dict:
    """All layer inputs for one workload.

    Layouts (row-major): u [T][d]; centroids [n][d]; w1, w3 [n][d_ff][d];
    w2 [n][d][d_ff]; shared dense view ws1, ws3 [K_s*d_ff][d], ws2 [d][K_s*d_ff]
    (shared expert q owns rows / columns q*d_ff .. (q+1)*d_ff - 1).
    bf16 tensors are uint16 bit patterns; fp32 tensors are float32.
    """
    n, d, f, ks = cfg.n, cfg.d, cfg.d_ff, cfg.K_s
    u, cent, redraws = make_router_inputs(cfg, seed, certify)
    w1 = _weights(_rng(seed, "w1"), n, f, d, cfg.w_std, cfg.dtype)
    w3 = _weights(_rng(seed, "w3"), n, f, d, cfg.w_std, cfg.dtype)
    w2 = _weights(_rng(seed, "w2"), n, d, f, cfg.w_std, cfg.dtype)
    if ks > 0:
        ws1 = _weights(_rng(seed, "ws1"), 1, ks * f, d, cfg.w_std, cfg.dtype)[0]
        ws3 = _weights(_rng(seed, "ws3"), 1, ks * f, d, cfg.w_std, cfg.dtype)[0]
        ws2 = _weights(_rng(seed, "ws2"), 1, d, ks * f, cfg.w_std, cfg.dtype)[0]
    else:
        ws1 = ws3 = ws2 = None
    return dict(cfg=cfg, seed=seed, u=u, centroids=cent, w1=w1, w3=w3, w2=w2,
                ws1=ws1, ws3=ws3, ws2=ws2, redraws=redraws)
