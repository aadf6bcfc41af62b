"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what it pins.  Sources: the DeepSeekMoE explainer page
(deepforge.srivtx.xyz "DeepSeekMoE"): the routing equation of section "Routing
in a classic MoE layer", the note under "Top-k routing, from affinities to
gates" (softmax over all experts before the cut, kept gates do not sum to
one), section "Expert-level balance loss", section "What the 16B configuration
looks like", question 5 of "Implementation check", and the stretch goals of
"Build it yourself" (router unit tests: ties, k equal to the number of experts,
a single-expert layer).  SwiGLU follows "GLU Variants Improve Transformer".
"""
import itertools
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import moe_synth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def silu(z):
    return z / (1.0 + math.exp(-z))


def f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def tiny_layer_inputs(u, cent, w1, w3, w2, ws1=None, ws3=None, ws2=None):
    return dict(u=f32(u), centroids=f32(cent), w1=f32(w1), w3=f32(w3), w2=f32(w2),
                ws1=None if ws1 is None else f32(ws1), ws3=None if ws3 is None else f32(ws3),
                ws2=None if ws2 is None else f32(ws2))


# ---------------------------------------------------------------- page facts

def test_page_printed_counts_and_shapes():
    """Pins the reading n = mN (routed), k = mK - K_s, with mK counting the
    shared experts: the 16B layer (16, 4, 2, K_s=2) keeps 6 routed experts and
    runs 8 expert passes; 8-of-64 gives the printed combination count."""
    g = json.load(open(GOLD))
    assert math.comb(16, 2) == g["combinations_2_of_16"]["value"]
    assert math.comb(64, 8) == g["combinations_8_of_64"]["value"]
    n, k = oracle.sizes(16, 4, 2, 2)
    b16 = g["16b"]
    assert (n, k) == (b16["routed"], b16["routed_active"])
    assert k + 2 == b16["expert_passes_per_token"]
    assert math.comb(n, k + 2) == g["combinations_8_of_64"]["value"]
    # the 2-of-16 baseline: N=16 experts, K=2 active, no segmentation
    n0, k0 = oracle.sizes(16, 1, 2, 0)
    assert math.comb(n0, k0) == g["combinations_2_of_16"]["value"]
    n1, k1 = oracle.sizes(32, 4, 4, 4)
    assert (n1, k1) == (g["145b"]["routed"], g["145b"]["routed_active"])
    # fine-grained experts are 1/m of the width: the 16B expert width is 1/4
    assert 1 / 4 == b16["expert_width_fraction"]
    cfg = moe_synth.CONFIGS["16b"]
    assert (cfg.n, cfg.k, cfg.K_s, cfg.d) == (64, 6, 2, b16["hidden"])
    assert (moe_synth.CONFIGS["145b"].n, moe_synth.CONFIGS["145b"].k,
            moe_synth.CONFIGS["145b"].K_s) == (128, 12, 4)
    with pytest.raises(ValueError):
        oracle.sizes(4, 1, 1, 1)   # k = 0
    with pytest.raises(ValueError):
        oracle.sizes(2, 1, 3, 0)   # k > n


# ---------------------------------------------------------------- routing

def test_two_expert_gates_are_sigmoid():
    """Closed form: with two experts the softmax is a sigmoid of the logit gap."""
    a, b = 0.75, -0.5
    u = [[1.0, 0.0]]
    cent = [[a, 0.0], [b, 0.0]]
    r = oracle.route(f32(u), f32(cent), 2)
    assert r["topk_idx"].tolist() == [[0, 1]]
    s0 = 1.0 / (1.0 + math.exp(b - a))
    np.testing.assert_allclose(r["topk_gate"][0], [s0, 1.0 - s0], rtol=1e-6)
    r1 = oracle.route(f32(u), f32(cent), 1)
    assert r1["topk_idx"].tolist() == [[0]]
    np.testing.assert_allclose(r1["topk_gate"][0, 0], s0, rtol=1e-6)
    # the larger-logit expert wins even when it has the higher index
    r2 = oracle.route(f32(u), f32([[b, 0.0], [a, 0.0]]), 1)
    assert r2["topk_idx"].tolist() == [[1]]


def test_softmax_large_logits_closed_form():
    """Softmax of (100, 99, 98) without overflow: 1, e^-1, e^-2 over their sum."""
    r = oracle.route(f32([[1.0]]), f32([[98.0], [100.0], [99.0]]), 3)
    assert r["topk_idx"].tolist() == [[1, 2, 0]]
    z = 1 + math.exp(-1) + math.exp(-2)
    np.testing.assert_allclose(r["topk_gate"][0], [1 / z, math.exp(-1) / z, math.exp(-2) / z],
                               rtol=1e-6)


def test_topk_set_and_order_brute_force():
    """Selected set = the k-subset with the largest logit sum (exhaustive
    search over all subsets); order = descending logit; gates = softmax values
    in fp64 (the Python sketch's precision)."""
    cfg = moe_synth.MoEConfig("t", T=40, d=12, N=7, m=1, K=3, K_s=0, d_ff=4, dtype="f32",
                              cent_std=0.5)
    u, c, _ = moe_synth.make_router_inputs(cfg, seed=3)
    r = oracle.route(u, c, cfg.k)
    lg = u.astype(np.float64) @ c.astype(np.float64).T
    for t in range(cfg.T):
        best = max(itertools.combinations(range(cfg.n), cfg.k),
                   key=lambda s: sum(lg[t, i] for i in s))
        got = r["topk_idx"][t].tolist()
        assert sorted(got) == sorted(best)
        assert all(lg[t, got[j]] > lg[t, got[j + 1]] for j in range(cfg.k - 1))
        s = np.exp(lg[t] - lg[t].max())
        s /= s.sum()
        np.testing.assert_allclose(r["topk_gate"][t], s[got], rtol=2e-5)
        assert r["topk_gate"][t].sum() < 1.0   # kept gates do not sum to one


def test_k_equals_n_gates_are_full_softmax():
    """k = n: the gates are the whole softmax, so they sum to one and are sorted."""
    cfg = moe_synth.MoEConfig("t", T=16, d=8, N=5, m=1, K=5, K_s=0, d_ff=4, dtype="f32",
                              cent_std=0.7)
    u, c, _ = moe_synth.make_router_inputs(cfg, seed=1)
    r = oracle.route(u, c, 5)
    for t in range(cfg.T):
        assert sorted(r["topk_idx"][t].tolist()) == list(range(5))
        g = r["topk_gate"][t].astype(np.float64)
        assert abs(g.sum() - 1.0) < 5 * 2.0 ** -23
        assert np.all(np.diff(g) <= 0)


def test_single_expert_layer():
    """n = 1: the gate is exactly one, and h = u + FFN_0(u)."""
    u = [[0.5, -1.0], [2.0, 0.25]]
    inp = tiny_layer_inputs(u, [[0.3, 0.1]], w1=[[[1.0, 0.0]]], w3=[[[0.0, 1.0]]],
                            w2=[[[1.0], [2.0]]])
    o = oracle.layer(inp, N=1, m=1, K=1, K_s=0)
    assert o["topk_gate"].tolist() == [[1.0], [1.0]]
    for t, (x0, x1) in enumerate(u):
        v = silu(x0) * x1
        np.testing.assert_allclose(o["h"][t], [x0 + v, x1 + 2 * v], rtol=1e-6, atol=1e-7)


def test_ties_go_to_lower_index():
    """Duplicate centroids: the stable order keeps the lower index first."""
    c = [[1.0, 0.0], [2.0, 0.0], [1.0, 0.0], [2.0, 0.0]]
    r = oracle.route(f32([[1.0, 3.0]]), f32(c), 3)
    assert r["topk_idx"].tolist() == [[1, 3, 0]]


def test_uniform_router_statistics_closed_form():
    """u = 0: every logit is 0, s_i = 1/n exactly (n a power of two), the tie
    rule picks experts 0..k-1 for every token, so counts = T there, f_i = n/k,
    P_i = 1/n and L_ExpBal = alpha * sum f P = alpha."""
    T, n, k = 64, 16, 4
    r = oracle.route(np.zeros((T, 8), np.float32),
                     moe_synth.as_f32(np.ones((n, 8), np.float32)), k)
    assert (r["topk_idx"] == np.arange(k)).all()
    assert r["counts"].tolist() == [T] * k + [0] * (n - k)
    assert r["f"].tolist() == [n / k] * k + [0.0] * (n - k)
    assert r["P"].tolist() == [1.0 / n] * n
    assert oracle.balance_loss(r["f"], r["P"], 0.001) == np.float32(0.001)


def test_balance_statistic_invariants():
    """sum counts = kT (exact), sum f = n, sum P = 1; f_i = count_i * n/(kT)."""
    cfg = moe_synth.CONFIGS["tiny"]
    inp = moe_synth.make_inputs(cfg)
    r = oracle.route(inp["u"], inp["centroids"], cfg.k, want_scores=True)
    assert int(r["counts"].sum()) == cfg.k * cfg.T
    assert np.bincount(r["topk_idx"].ravel(), minlength=cfg.n).tolist() == r["counts"].tolist()
    assert abs(float(r["f"].astype(np.float64).sum()) - cfg.n) < 1e-4
    assert abs(float(r["P"].astype(np.float64).sum()) - 1.0) < 1e-5
    np.testing.assert_allclose(r["f"], r["counts"] * cfg.n / (cfg.k * cfg.T), rtol=1e-7)
    np.testing.assert_allclose(r["P"], r["scores"].astype(np.float64).mean(axis=0), rtol=1e-5)
    # a balanced router gives L = alpha: f = 1, P = 1/n
    assert abs(oracle.balance_loss(np.ones(16, np.float32), np.full(16, 1 / 16, np.float32),
                                   0.01) - 0.01) < 1e-9


# ---------------------------------------------------------------- permutation

def test_permute_equals_stable_argsort():
    """The grouping is a stable sort of the (token, slot) pairs by expert."""
    rng = np.random.default_rng(5)
    T, n, k = 300, 13, 4
    idx = np.stack([rng.permutation(n)[:k] for _ in range(T)]).astype(np.int32)
    p = oracle.permute(idx, n)
    order = np.argsort(idx.ravel(), kind="stable")
    assert (p["perm_token"] == order // k).all()
    slot = np.empty(T * k, np.int64)
    slot[order] = np.arange(T * k)
    assert (p["slot_of"].ravel() == slot).all()
    assert (p["offsets"] == np.concatenate([[0], np.cumsum(np.bincount(idx.ravel(),
                                                                       minlength=n))])).all()


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_closed_form_and_branches():
    """FFN(x) = W2 (SiLU(W1 x) * (W3 x)); sigmoid(ln 3) = 3/4 gives
    SiLU(ln 3) = 0.75 ln 3 exactly in closed form."""
    x = f32([1.0, 0.0])
    w1 = f32([[[math.log(3.0), 0.0]]])
    w3 = f32([[[2.0, 0.0]]])
    w2 = f32([[[1.0], [-0.5]]])
    y = oracle.expert(x, 0, w1, w3, w2)
    v = 0.75 * math.log(3.0) * 2.0
    np.testing.assert_allclose(y, [v, -0.5 * v], rtol=1e-6)
    # the SiLU sits on the W1 branch: a very negative W1 x silences the expert
    y = oracle.expert(x, 0, f32([[[-40.0, 0.0]]]), w3, w2)
    assert np.abs(y).max() < 1e-14
    # W1 x = 0 gives exactly zero
    assert (oracle.expert(x, 0, f32([[[0.0, 1.0]]]), w3, w2) == 0).all()
    # linear in W3 and W2 (exact for a power-of-two scale), not in W1
    rng = np.random.default_rng(0)
    W1, W3, W2 = (f32(rng.normal(size=s)) for s in [(1, 3, 5), (1, 3, 5), (1, 5, 3)])
    xx = f32(rng.normal(size=5))
    base = oracle.expert(xx, 0, W1, W3, W2)
    assert (oracle.expert(xx, 0, W1, 2 * W3, W2) == 2 * base).all()
    assert (oracle.expert(xx, 0, W1, W3, 2 * W2) == 2 * base).all()
    assert not np.allclose(oracle.expert(xx, 0, 2 * W1, W3, W2), 2 * base)


def test_swiglu_orientation_one_hot():
    """One-hot weights with d != d_ff pin the operand orientation:
    W1[c=1][j=2] = W3[c=1][j=0] = W2[i=1][c=1] = 1 gives y = (0, SiLU(x2) x0, 0)."""
    d, d_ff, n, e = 3, 2, 2, 1
    w1 = np.zeros((n, d_ff, d), np.float32)
    w3 = np.zeros((n, d_ff, d), np.float32)
    w2 = np.zeros((n, d, d_ff), np.float32)
    w1[e, 1, 2] = w3[e, 1, 0] = w2[e, 1, 1] = 1.0
    x = f32([0.7, -1.3, 0.4])
    y = oracle.expert(x, e, w1, w3, w2)
    np.testing.assert_allclose(y, [0.0, silu(0.4) * 0.7, 0.0], rtol=1e-6)
    assert (oracle.expert(x, 0, w1, w3, w2) == 0).all()   # expert 0 is all zero


# ---------------------------------------------------------------- whole layer

def _designed_two_expert_inputs(x, with_shared):
    """d = 2, d_ff = 1.  Centroids e0 = (1, 0), e1 = (0, 1): the logits are
    the coordinates.  FFN_0(u) = (SiLU(u0) u1, 0), FFN_1(u) = (0, SiLU(u1) u0);
    shared expert S(u) = (0, SiLU(u1) u1)."""
    w1 = [[[1.0, 0.0]], [[0.0, 1.0]]]
    w3 = [[[0.0, 1.0]], [[1.0, 0.0]]]
    w2 = [[[1.0], [0.0]], [[0.0], [1.0]]]
    sh = dict(ws1=[[0.0, 1.0]], ws3=[[0.0, 1.0]], ws2=[[0.0], [1.0]]) if with_shared else {}
    return tiny_layer_inputs([x], [[1.0, 0.0], [0.0, 1.0]], w1, w3, w2, **sh)


@pytest.mark.parametrize("x", [(1.0, 0.5), (-0.25, 0.75)])
def test_layer_closed_form_gshard_top1(x):
    """m = 1, K_s = 0 (GShard top-K of N): h = u + s_sel FFN_sel(u)."""
    x0, x1 = x
    o = oracle.layer(_designed_two_expert_inputs(x, False), N=2, m=1, K=1, K_s=0)
    s0 = 1.0 / (1.0 + math.exp(x1 - x0))
    if x0 > x1:
        want = [x0 + s0 * silu(x0) * x1, x1]
    else:
        want = [x0, x1 + (1 - s0) * silu(x1) * x0]
    np.testing.assert_allclose(o["h"][0], want, rtol=1e-6)
    np.testing.assert_allclose(o["ysum"][0], np.array(want) - np.array(x), rtol=1e-6, atol=1e-7)


def test_layer_closed_form_all_experts_plus_shared():
    """k = n = 2 with one shared expert that has no centroid and weight one:
    h = u + s0 FFN_0 + s1 FFN_1 + S; (N, m, K, K_s) = (2, 1, 3, 1)."""
    x0, x1 = 0.3, -0.6
    o = oracle.layer(_designed_two_expert_inputs((x0, x1), True), N=2, m=1, K=3, K_s=1)
    s0 = 1.0 / (1.0 + math.exp(x1 - x0))
    want = [x0 + s0 * silu(x0) * x1, x1 + (1 - s0) * silu(x1) * x0 + silu(x1) * x1]
    np.testing.assert_allclose(o["h"][0], want, rtol=1e-6)
    np.testing.assert_allclose(o["S"][0], [0.0, silu(x1) * x1], rtol=1e-6)
    assert o["topk_gate"][0].sum() == pytest.approx(1.0, abs=1e-7)


def test_layer_equals_dense_masked_evaluation():
    """Brute force: evaluate every routed expert on every token and weight it
    by a 0/1 top-k mask times s_i (mask from exhaustive subset search)."""
    cfg = moe_synth.MoEConfig("t", T=12, d=8, N=6, m=1, K=3, K_s=1, d_ff=4, dtype="f32",
                              cent_std=0.6, w_std=0.3)
    inp = moe_synth.make_inputs(cfg, seed=2)
    o = oracle.layer(inp, cfg.N, cfg.m, cfg.K, cfg.K_s)
    r = oracle.route(inp["u"], inp["centroids"], cfg.k, want_scores=True)
    lg = inp["u"].astype(np.float64) @ inp["centroids"].astype(np.float64).T
    for t in range(cfg.T):
        best = set(max(itertools.combinations(range(cfg.n), cfg.k),
                       key=lambda s: sum(lg[t, i] for i in s)))
        acc = np.zeros(cfg.d)
        for i in range(cfg.n):
            mask = 1.0 if i in best else 0.0
            acc += mask * r["scores"][t, i] * oracle.expert(inp["u"][t], i, inp["w1"], inp["w3"],
                                                            inp["w2"])
        # the shared expert as a routed-layout expert with weight one
        sw1 = inp["ws1"][None]
        sw3 = inp["ws3"][None]
        sw2 = inp["ws2"][None]
        acc += oracle.expert(inp["u"][t], 0, sw1, sw3, sw2)
        np.testing.assert_allclose(o["h"][t], acc + inp["u"][t], rtol=1e-5, atol=1e-6)


def test_shared_experts_equal_one_dense_swiglu():
    """K_s shared experts = one SwiGLU whose hidden layer is their
    concatenation: with the routed output zeroed (W2 = 0), the layer with two
    shared experts of width f matches the layer with one of width 2f."""
    f = 3
    base = moe_synth.MoEConfig("t", T=10, d=6, N=4, m=1, K=4, K_s=2, d_ff=f, dtype="f32",
                               cent_std=0.5, w_std=0.4)
    inp = moe_synth.make_inputs(base, seed=4)
    inp["w2"] = np.zeros_like(inp["w2"])
    a = oracle.layer(inp, 4, 1, 4, 2)            # k = 2, shared split in two
    inp2 = dict(inp)
    inp2["w1"] = np.zeros((4, 2 * f, 6), np.float32)
    inp2["w3"] = np.zeros((4, 2 * f, 6), np.float32)
    inp2["w2"] = np.zeros((4, 6, 2 * f), np.float32)
    b = oracle.layer(inp2, 4, 1, 3, 1)           # k = 2, one shared of width 2f
    assert (a["topk_idx"] == b["topk_idx"]).all()
    np.testing.assert_allclose(a["S"], b["S"], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(a["h"], b["h"], rtol=1e-6, atol=1e-7)
    # and each shared expert is a routed-layout expert on its slice
    x = inp["u"][0]
    s_manual = sum(oracle.expert(x, 0, inp["ws1"][q * f:(q + 1) * f][None],
                                 inp["ws3"][q * f:(q + 1) * f][None],
                                 np.ascontiguousarray(inp["ws2"][:, q * f:(q + 1) * f])[None])
                   for q in range(2))
    np.testing.assert_allclose(a["S"][0], s_manual, rtol=1e-6, atol=1e-7)


def test_factorisation_invariance():
    """Only mN and mK - K_s enter: (16,4,2), (64,1,8), (8,8,1) with K_s = 2 give
    bit-identical layers."""
    cfg = moe_synth.MoEConfig("t", T=24, d=16, N=16, m=4, K=2, K_s=2, d_ff=8, dtype="f32",
                              cent_std=0.3, w_std=0.2)
    inp = moe_synth.make_inputs(cfg, seed=7)
    outs = [oracle.layer(inp, N, m, K, 2) for (N, m, K) in [(16, 4, 2), (64, 1, 8), (8, 8, 1)]]
    for o in outs[1:]:
        for key in ("topk_idx", "topk_gate", "counts", "f", "P", "h", "Y", "S"):
            assert (o[key] == outs[0][key]).all(), key


def test_subset_tokens_match_full_layer():
    """The token-subset entry returns exactly the full run's rows."""
    cfg = moe_synth.CONFIGS["tiny"]
    inp = moe_synth.make_inputs(cfg)
    full = oracle.layer(inp, cfg.N, cfg.m, cfg.K, cfg.K_s)
    toks = np.array([63, 0, 17], np.int64)
    sub = oracle.layer(inp, cfg.N, cfg.m, cfg.K, cfg.K_s, toks=toks)
    for key in ("h", "Y", "S", "ysum"):
        assert (sub[key] == full[key][toks]).all()


def test_oracle_thread_count_invariance():
    """Results are bit-identical with 1 and 4 OpenMP threads."""
    code = ("import sys,hashlib; sys.path.insert(0, %r); import moe_synth, oracle; "
            "c = moe_synth.CONFIGS['tiny']; i = moe_synth.make_inputs(c); "
            "o = oracle.layer(i, c.N, c.m, c.K, c.K_s); "
            "print(hashlib.sha256(b''.join(o[k].tobytes() for k in sorted(o))).hexdigest())"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    outs = []
    for nthr in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=nthr)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True, text=True).stdout.strip())
    assert outs[0] == outs[1]


def test_bf16_storage_is_widened_exactly():
    """bf16 bits are read as the exact fp32 value: a bf16 run equals the fp32
    run on the widened values."""
    cfg = moe_synth.MoEConfig("t", T=8, d=32, N=4, m=2, K=2, K_s=1, d_ff=32, dtype="bf16")
    inp = moe_synth.make_inputs(cfg, seed=1)
    wide = {k: (moe_synth.as_f32(v) if isinstance(v, np.ndarray) and v.dtype == np.uint16 else v)
            for k, v in inp.items()}
    a = oracle.layer(inp, cfg.N, cfg.m, cfg.K, cfg.K_s)
    b = oracle.layer(wide, cfg.N, cfg.m, cfg.K, cfg.K_s)
    for key in ("topk_idx", "topk_gate", "h"):
        assert (a[key] == b[key]).all()


def test_combine_closed_form():
    """h = sum_j g_j y[slot_j] + shared + residual with exact small values."""
    y = f32([[2.0, 4.0], [8.0, -2.0], [1.0, 1.0]])
    slot = np.array([[2, 0], [1, 2]], np.int32)
    gate = f32([[0.5, 0.25], [0.125, 1.0]])
    sh = f32([[1.0, 0.0], [0.0, 1.0]])
    res = f32([[10.0, 20.0], [30.0, 40.0]])
    h = oracle.combine(y, slot, gate, sh, res)
    want = [[0.5 * 1 + 0.25 * 2 + 1 + 10, 0.5 * 1 + 0.25 * 4 + 0 + 20],
            [0.125 * 8 + 1 * 1 + 0 + 30, 0.125 * -2 + 1 * 1 + 1 + 40]]
    assert h.tolist() == want
    h2 = oracle.combine(y, slot, gate)
    assert h2.tolist() == (np.array(want) - sh - res).tolist()


def test_combine_matches_layer():
    """The combine entry reproduces the layer's h from its own Y and S."""
    cfg = moe_synth.CONFIGS["tiny"]
    inp = moe_synth.make_inputs(cfg)
    o = oracle.layer(inp, cfg.N, cfg.m, cfg.K, cfg.K_s)
    pm = oracle.permute(o["topk_idx"], cfg.n)
    y_perm = np.empty((cfg.T * cfg.k, cfg.d), np.float32)
    y_perm[pm["slot_of"].ravel()] = o["Y"].reshape(-1, cfg.d)
    h = oracle.combine(y_perm, pm["slot_of"], o["topk_gate"], o["S"], inp["u"])
    assert (h == o["h"]).all()


def test_granularity_sweep_keeps_the_budget():
    """The granularity sweep cuts the 16B shape's 16 experts of width 5632
    (2 active) into m finer ones: total and activated expert widths stay the
    same, and m = 1 with no shared experts is GShard's top-2 layer."""
    g = moe_synth.GRANULARITY
    assert sorted(c.m for c in g.values()) == [1, 2, 4, 8]
    for c in g.values():
        assert c.K_s == 0 and c.N == 16 and c.K == 2 and c.d == 2048
        assert c.n * c.d_ff == 16 * 5632      # all experts
        assert c.k * c.d_ff == 2 * 5632       # experts a token passes through
        assert c.n == 16 * c.m and c.k == 2 * c.m
    m1 = g["gran_m1"]
    assert (m1.n, m1.k, m1.K_s) == (16, 2, 0)
    # at m = 4 the fine experts have the 16B shape's width
    assert g["gran_m4"].d_ff == moe_synth.CONFIGS["16b"].d_ff
