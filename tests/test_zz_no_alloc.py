"""moe_layer_fwd_noalloc (no caller workspace: the library's fixed per-device
scratch array) against moe_layer_fwd on a caller workspace: the same kernels,
so the same bits.  Two calls in a row, the second on a smaller problem, so
the second runs on the scratch the first left behind."""
import numpy as np
import pytest

import moe_synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_34_amd as moe
    from mixture_experts_layer_34_amd.device import to_device, workspace

# the 16B shape at 64 tokens (the decode regime), then a smaller layer
# with ragged tiles that takes the tiled GEMM on row-major weights
CASES = [
    (moe_synth.CONFIGS["16b_decode"], True),
    (moe_synth.MoEConfig("small", T=40, d=224, N=16, m=1, K=4, K_s=1, d_ff=160, dtype="bf16"),
     False),
]


def run(cfg, packed, noalloc):
    d = "cuda"
    inp = moe_synth.make_inputs(cfg, seed=0)
    p = moe.problem(cfg.T, cfg.d, cfg.N, cfg.m, cfg.K, cfg.K_s, cfg.d_ff, cfg.dtype)
    t = {k: to_device(inp[k], d) for k in ("u", "centroids", "w1", "w3", "w2", "ws1", "ws3",
                                           "ws2")}
    if packed:
        for k in ("w1", "w3", "w2", "ws1", "ws3", "ws2"):
            dst = torch.empty_like(t[k])
            moe.moe_pack_weights(p, t[k].numel() // t[k].shape[-1], t[k].shape[-1], t[k], dst)
            t[k] = dst
    out = dict(h=torch.full((cfg.T, cfg.d), -7.0, dtype=torch.bfloat16, device=d),
               idx=torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device=d),
               gate=torch.full((cfg.T, cfg.k), -7.0, dtype=torch.float32, device=d),
               counts=torch.full((cfg.n,), -7, dtype=torch.int32, device=d),
               f=torch.full((cfg.n,), -7.0, dtype=torch.float32, device=d),
               P=torch.full((cfg.n,), -7.0, dtype=torch.float32, device=d))
    args = (p, t["u"], t["centroids"], t["w1"], t["w3"], t["w2"], t["ws1"], t["ws3"], t["ws2"],
            out["h"], out["idx"], out["gate"], out["counts"], out["f"], out["P"],
            moe.MOE_PACKED_WEIGHTS if packed else 0)
    if noalloc:
        moe.moe_layer_fwd_noalloc(*args)
    else:
        ws = workspace(p, d)
        ws.fill_(0x5A)
        moe.moe_layer_fwd(*args, ws)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def test_noalloc_matches_layer_fwd_twice_second_smaller():
    for cfg, packed in CASES:
        p = moe.problem(cfg.T, cfg.d, cfg.N, cfg.m, cfg.K, cfg.K_s, cfg.d_ff, cfg.dtype)
        assert moe.moe_workspace_bytes(p) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        print(f"noalloc {cfg.name} T={cfg.T} d={cfg.d} n={cfg.n} packed={packed}", flush=True)
        got = run(cfg, packed, True)
        want = run(cfg, packed, False)
        for k in want:
            assert torch.equal(got[k], want[k]), (cfg.name, k)


def test_noalloc_rejects_problems_beyond_its_scratch():
    cfg = moe_synth.CONFIGS["16b"]
    p = moe.problem(cfg.T, cfg.d, cfg.N, cfg.m, cfg.K, cfg.K_s, cfg.d_ff, cfg.dtype)
    assert moe.moe_workspace_bytes(p) > moe.MOE_NOALLOC_SCRATCH_BYTES
    A = 0x100000
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_fwd_noalloc(p, *([A] * 14), 0)
    assert "WORKSPACE" in str(ei.value)
