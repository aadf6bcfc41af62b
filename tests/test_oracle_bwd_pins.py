"""Pins of the oracle's backward pass to facts that do not come from it.

The quantity differentiated is L = sum_t <dh_t, h_t> + alpha * sum_i f_i P_i:
the layer of the DeepSeekMoE explainer (deepforge.srivtx.xyz "DeepSeekMoE",
section "Routing in a classic MoE layer") contracted with an upstream
gradient, plus the expert-level balance loss of section "Expert-level balance
loss".  The kept sets and the counts behind f_i are constant near a point
whose logits have no near-ties at the cut, so L is smooth there and its
gradient is fixed by central finite differences of an independent fp64
forward written below with numpy.  Further pins: the balance term's gradient
vanishes for uniform f (the softmax sums to one), linearity in (dh, alpha),
and consistency of the oracle's token and expert subsets with the full run.
"""
import numpy as np
import pytest

import moe_synth
import oracle


def bits_to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def silu64(z):
    return z / (1.0 + np.exp(-z))


def loss64(x, idx, f, dh, alpha, n_shared, d_ff, residual=True):
    """Independent fp64 forward of L with the kept sets idx held fixed.
    x: dict of fp64 arrays u, centroids, w1, w3, w2 (+ ws1, ws3, ws2)."""
    u, c = x["u"], x["centroids"]
    lg = u @ c.T
    lg = lg - lg.max(axis=1, keepdims=True)
    s = np.exp(lg)
    s = s / s.sum(axis=1, keepdims=True)
    T = u.shape[0]
    h = u.copy() if residual else np.zeros_like(u)
    for t in range(T):
        for e in idx[t]:
            a = x["w1"][e] @ u[t]
            b = x["w3"][e] @ u[t]
            h[t] += s[t, e] * (x["w2"][e] @ (silu64(a) * b))
        for q in range(n_shared):
            sl = slice(q * d_ff, (q + 1) * d_ff)
            a = x["ws1"][sl] @ u[t]
            b = x["ws3"][sl] @ u[t]
            h[t] += x["ws2"][:, sl] @ (silu64(a) * b)
    P = s.mean(axis=0)
    return float((dh * h).sum() + alpha * (f * P).sum())


def make_case(T, d, N, m, K, K_s, d_ff, dtype, seed):
    """Tiny inputs whose logits keep a clear gap at the top-k cut."""
    n, k = oracle.sizes(N, m, K, K_s)
    rng = np.random.default_rng(seed)
    for _ in range(50):
        raw = dict(u=rng.normal(0, 1.0, (T, d)), centroids=rng.normal(0, 0.6, (n, d)),
                   w1=rng.normal(0, 0.4, (n, d_ff, d)), w3=rng.normal(0, 0.4, (n, d_ff, d)),
                   w2=rng.normal(0, 0.4, (n, d, d_ff)))
        if K_s:
            raw.update(ws1=rng.normal(0, 0.4, (K_s * d_ff, d)),
                       ws3=rng.normal(0, 0.4, (K_s * d_ff, d)),
                       ws2=rng.normal(0, 0.4, (d, K_s * d_ff)))
        if dtype == "bf16":
            inp = {kk: moe_synth.f32_to_bf16_bits(v.astype(np.float32)) for kk, v in raw.items()}
        else:
            inp = {kk: np.ascontiguousarray(v, np.float32) for kk, v in raw.items()}
        x = {kk: bits_to_f64(v) for kk, v in inp.items()}
        lg = np.sort(x["u"] @ x["centroids"].T, axis=1)[:, ::-1]
        gap = (lg[:, k - 1] - lg[:, k]).min() if k < n else np.inf
        if gap > 1e-2:
            break
    else:
        raise AssertionError("no draw with a clear top-k gap")
    if K_s == 0:
        for kk in ("ws1", "ws3", "ws2"):
            inp[kk] = None
    r = oracle.route(inp["u"], inp["centroids"], k)
    dh = rng.normal(0, 1.0, (T, d)).astype(np.float32)
    return inp, x, r, dh, n, k


CASES = {
    # routed + 2 shared experts, fp32 storage
    "f32_shared": dict(T=5, d=12, N=4, m=2, K=2, K_s=2, d_ff=6, dtype="f32"),
    # bf16 storage, no shared experts, every token keeps 3 of 6
    "bf16_routed": dict(T=6, d=8, N=3, m=2, K=3, K_s=0, d_ff=5, dtype="bf16"),
    # k = n: every expert kept
    "f32_all_kept": dict(T=4, d=8, N=3, m=1, K=3, K_s=0, d_ff=4, dtype="f32"),
}


def fd_grad(fn, arr, h=1e-5):
    g = np.empty_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h
        lp = fn()
        arr[i] = old - h
        lm = fn()
        arr[i] = old
        g[i] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("flags", [0, oracle.BWD_NO_RESIDUAL | oracle.BWD_NO_SHARED])
def test_bwd_matches_finite_differences(name, flags):
    """Every gradient the oracle forms equals the central difference of an
    independent fp64 forward of L, element by element."""
    c = CASES[name]
    inp, x, r, dh, n, k = make_case(c["T"], c["d"], c["N"], c["m"], c["K"], c["K_s"],
                                    c["d_ff"], c["dtype"], seed=3)
    alpha = 0.37
    f = r["f"].astype(np.float64)
    K_s = 0 if flags & oracle.BWD_NO_SHARED else c["K_s"]
    residual = not (flags & oracle.BWD_NO_RESIDUAL)
    dh64 = dh.astype(np.float64)
    fn = lambda: loss64(x, r["topk_idx"], f, dh64, alpha, K_s, c["d_ff"], residual)
    got = oracle.layer_bwd(inp, c["N"], c["m"], c["K"], c["K_s"], r["topk_idx"], r["f"], dh,
                           alpha, flags=flags, experts=np.arange(n))
    pairs = [("du", "u"), ("dcent", "centroids"), ("dw1", "w1"), ("dw3", "w3"), ("dw2", "w2")]
    if K_s:
        pairs += [("dws1", "ws1"), ("dws3", "ws3"), ("dws2", "ws2")]
    else:
        assert "dws1" not in got
    for gk, xk in pairs:
        want = fd_grad(fn, x[xk])
        err = np.abs(got[gk] - want).max()
        scale = max(1.0, np.abs(want).max())
        assert err <= 2e-6 * scale, (gk, err, scale)


def test_balance_gradient_vanishes_for_uniform_f():
    """With dh = 0 only the balance term is left; for equal f_i it is a
    multiple of sum_i P_i = 1, whose gradient is zero."""
    inp, x, r, dh, n, k = make_case(5, 12, 4, 2, 2, 1, 6, "f32", seed=5)
    f = np.full(n, 1.5, np.float32)
    got = oracle.layer_bwd(inp, 4, 2, 2, 1, r["topk_idx"], f, np.zeros_like(dh), 0.9,
                           flags=oracle.BWD_NO_RESIDUAL, experts=np.arange(n))
    for kk, v in got.items():
        assert np.abs(v).max() < 1e-12, kk
    # with non-uniform f the same call moves u and the centroids, not the weights
    got = oracle.layer_bwd(inp, 4, 2, 2, 1, r["topk_idx"], r["f"], np.zeros_like(dh), 0.9,
                           flags=oracle.BWD_NO_RESIDUAL, experts=np.arange(n))
    assert np.abs(got["du"]).max() > 1e-4 and np.abs(got["dcent"]).max() > 1e-4
    for kk in ("dw1", "dw3", "dw2", "dws1", "dws3", "dws2"):
        assert np.abs(got[kk]).max() == 0.0, kk


def test_bwd_is_linear_in_dh_and_alpha():
    inp, x, r, dh, n, k = make_case(6, 12, 4, 2, 2, 1, 6, "bf16", seed=7)
    rng = np.random.default_rng(8)
    # multiples of 2^-8: dh + dh2 is exact in fp32
    dh = (np.round(dh * 256) / 256).astype(np.float32)
    dh2 = (np.round(rng.normal(0, 1, dh.shape) * 256) / 256).astype(np.float32)
    run = lambda g, a: oracle.layer_bwd(inp, 4, 2, 2, 1, r["topk_idx"], r["f"], g, a,
                                        experts=np.arange(n))
    g1, g2, g12 = run(dh, 0.3), run(dh2, 0.5), run(dh + dh2, 0.8)
    for kk in g12:
        assert np.allclose(g1[kk] + g2[kk], g12[kk], rtol=1e-10, atol=1e-10), kk


def test_subsets_match_the_full_run():
    """du rows for a token list, with and without the centroid gradient, and
    weight gradients for an expert list, equal the same entries of the full run."""
    inp, x, r, dh, n, k = make_case(7, 8, 4, 2, 2, 1, 4, "f32", seed=9)
    full = oracle.layer_bwd(inp, 4, 2, 2, 1, r["topk_idx"], r["f"], dh, 0.2,
                            experts=np.arange(n))
    toks = np.array([5, 0, 3])
    for want_dcent in (False, True):
        sub = oracle.layer_bwd(inp, 4, 2, 2, 1, r["topk_idx"], r["f"], dh, 0.2, toks=toks,
                               want_dcent=want_dcent, experts=np.array([6, 1]),
                               want_shared=False)
        np.testing.assert_array_equal(sub["du"], full["du"][toks])
        for kk in ("dw1", "dw3", "dw2"):
            np.testing.assert_array_equal(sub[kk], full[kk][[6, 1]])
        assert "dws1" not in sub
    # an expert no token kept has zero weight gradients
    unused = sorted(set(range(n)) - set(r["topk_idx"].ravel().tolist()))
    for e in unused:
        assert np.abs(full["dw1"][e]).max() == 0.0 and np.abs(full["dw2"][e]).max() == 0.0
