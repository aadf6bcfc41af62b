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
    bad = moe_synth.margin_violations(moe_synth.as_f32(u), moe_synth.as_f32(c), cfg.k)
    assert not bad.any()
    assert redraws < cfg.T // 20 + 2
