"""Seeded input generator: determinism, bf16 rounding, margin certificate."""
import numpy as np
import pytest

import moe_synth


def test_bf16_round_to_nearest_even():
    one = 1.0
    vals = np.array([one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -9,
                     -2.5, 3.0e38, 2.0 ** -130], np.float32)
    got = moe_synth.bf16_bits_to_f32(moe_synth.f32_to_bf16_bits(vals))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    want = [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5, 2.9999e38, 2.0 ** -130]
    np.testing.assert_allclose(got[:5], want[:5], rtol=0)
    assert abs(got[5] - 3.0e38) / 3.0e38 < 2.0 ** -8
    assert got[6] == np.float32(2.0 ** -130)


def test_deterministic():
    cfg = moe_synth.CONFIGS["tiny"]
    a = moe_synth.make_inputs(cfg, seed=0)
    b = moe_synth.make_inputs(cfg, seed=0)
    c = moe_synth.make_inputs(cfg, seed=1)
    for k in ("u", "centroids", "w1", "w3", "w2", "ws1", "ws3", "ws2"):
        assert (a[k] == b[k]).all()
    assert not (a["u"] == c["u"]).all()


def test_zipf_scale():
    r = moe_synth.zipf_row_scale(128, 1.1)
    assert abs(r.mean() - 1.0) < 1e-12
    assert 28.5 < r[0] < 29.5 and 0.13 < r[-1] < 0.15
    assert np.all(np.diff(r) < 0)


@pytest.mark.parametrize("name", list(moe_synth.CONFIGS))
def test_router_inputs_are_certified(name):
    cfg = moe_synth.CONFIGS[name]
    u, c, redraws = moe_synth.make_router_inputs(cfg, seed=0)
    assert u.shape == (cfg.T, cfg.d) and c.shape == (cfg.n, cfg.d)
    assert u.dtype == (np.uint16 if cfg.dtype == "bf16" else np.float32)
    u32, c32 = moe_synth.as_f32(u), moe_synth.as_f32(c)
    margin = moe_synth.certified_margin(cfg.d, moe_synth.max_abs_logit(u32, c32))
    assert margin >= 1e-4
    assert not moe_synth.margin_violations(u32, c32, cfg.k, margin).any()
    # the Zipf-scaled router has logits near 100, so its margin is ~35x the
    # floor and about a third of its tokens are redrawn; the others far fewer
    assert redraws < (cfg.T // 2 if cfg.zipf_s else cfg.T // 20 + 2)


def test_certified_margin_formula():
    eps = 2.0 ** -24
    assert moe_synth.certified_margin(64, 0.5) == 1e-4
    assert moe_synth.certified_margin(4096, 100.0) == pytest.approx(8 * eps * 64 * 100.0)


def test_tie_pairs_are_exact_twins_and_certified():
    """Duplicated centroid rows give exactly tied logits; the certificate
    skips those gaps (the tie rule decides) and checks every other one."""
    cfg = moe_synth.MoEConfig("t", T=200, d=128, N=16, m=1, K=4, K_s=1, d_ff=64,
                              dtype="bf16", tie_pairs=True)
    u, c, _ = moe_synth.make_router_inputs(cfg, seed=0)
    assert np.array_equal(c[1::2], c[0::2])
    g = moe_synth.twin_groups(moe_synth.as_f32(c))
    assert np.array_equal(g[0::2], g[1::2]) and len(set(g.tolist())) == cfg.n // 2
    u32, c32 = moe_synth.as_f32(u), moe_synth.as_f32(c)
    assert not moe_synth.margin_violations(u32, c32, cfg.k).any()
    # the same tokens against centroids without twins: the zero gaps count
    lg = u32.astype(np.float64) @ c32.astype(np.float64).T
    assert (lg[:, 0::2] == lg[:, 1::2]).all()


def test_flat_router_ties_every_expert_and_the_oracle_keeps_the_lowest():
    """All-zero centroids: every logit is exactly 0, the whole row is one twin
    group (no redraw), and the oracle's selection rule (larger logit, then
    lower index) keeps experts 0 .. k-1 in that order with the uniform
    softmax 1/n as gates; counts, f and P follow in closed form."""
    import oracle
    cfg = moe_synth.MoEConfig("f", T=70, d=64, N=8, m=2, K=2, K_s=1, d_ff=32,
                              dtype="bf16", flat_router=True)
    u, c, redraws = moe_synth.make_router_inputs(cfg, seed=0)
    assert redraws == 0 and not moe_synth.as_f32(c).any()
    r = oracle.route(u, c, cfg.k)
    assert (r["topk_idx"] == np.arange(cfg.k)[None, :]).all()
    assert np.allclose(r["topk_gate"], 1.0 / cfg.n, rtol=0, atol=1e-7)
    want = np.zeros(cfg.n, np.int64)
    want[:cfg.k] = cfg.T
    assert np.array_equal(r["counts"], want)
    assert np.allclose(r["f"], want * cfg.n / (cfg.k * cfg.T), rtol=1e-6)
    assert np.allclose(r["P"], 1.0 / cfg.n, rtol=1e-5)


def test_margin_violation_is_detected():
    """Two experts whose logits differ by less than the margin for one token."""
    u = np.zeros((2, 32), np.float32)
    u[:, 0] = 1.0
    c = np.zeros((3, 32), np.float32)
    c[0, 0], c[1, 0], c[2, 0] = 1.0, 1.0 + 5e-5, -1.0
    u[1, 1] = 1.0
    c[1, 1] = 1.0  # token 1 sees expert 1 a full unit above expert 0
    bad = moe_synth.margin_violations(u, c, 1)
    assert bad.tolist() == [True, False]
