"""GPU parity of every entry point against the CPU oracle.

Each component gets inputs derived from the oracle (never from the GPU path)
so a failure names one kernel: routing (bit-exact indices, counts, f),
grouping (bit-exact), the grouped SwiGLU FFN (per-slot, ungated), the
shared experts as one dense group, the combine, and the fused layer.
Every workload compares every token: routing outputs, per-slot expert
outputs, the shared sum and the layer output.
"""
import numpy as np
import pytest

import moe_synth
import oracle
from gpu_helpers import ALL, FULL, REL_TOL, elem_rel, gate_tol, inputs, p_tol, rel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_34_amd as moe
    from mixture_experts_layer_34_amd.device import to_device, torch_dtype, workspace

NAMES = list(ALL)
DECODE = [n for n in NAMES if n.startswith("decode")]
EDGE = [n for n in NAMES if ALL[n].tie_pairs or ALL[n].flat_router or ALL[n].n == 1]


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


def prob(cfg):
    return moe.problem(cfg.T, cfg.d, cfg.N, cfg.m, cfg.K, cfg.K_s, cfg.d_ff, cfg.dtype)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def exact_tol(cfg):
    """fp32 workloads run the whole path in fp32: hold them to 1e-4."""
    return 1e-4 if cfg.dtype == "f32" else REL_TOL


class Case:
    """One workload: seeded inputs, oracle results and device copies, built
    once per module run."""

    def __init__(self, name):
        self.name = name
        self.cfg = cfg = ALL[name]
        self.inp = inputs(name)
        r = oracle.route(self.inp["u"], self.inp["centroids"], cfg.k, want_scores=True)
        self.max_abs_logit = float(np.abs(r.pop("logits")).max())
        r.pop("scores")
        self.route = r
        self.perm = oracle.permute(r["topk_idx"], cfg.n)
        self.toks = np.arange(cfg.T)
        self.layer = oracle.layer(self.inp, cfg.N, cfg.m, cfg.K, cfg.K_s)
        self.dev = {k: to_device(self.inp[k], "cuda")
                    for k in ("u", "centroids", "w1", "w3", "w2", "ws1", "ws3", "ws2")}
        self._packed = None

    def weights(self, packed):
        """Row-major weights, or their packed copies (bf16 only)."""
        if not packed:
            return self.dev
        if self._packed is None:
            self._packed = dict(self.dev)
            p = prob(self.cfg)
            for k in ("w1", "w3", "w2", "ws1", "ws3", "ws2"):
                t = self.dev[k]
                if t is None:
                    continue
                rows, K = t.numel() // t.shape[-1], t.shape[-1]
                out = torch.empty_like(t)
                moe.moe_pack_weights(p, rows, K, t, out)
                self._packed[k] = out
            torch.cuda.synchronize()
        return self._packed


def packed_flag(case, packed):
    return moe.MOE_PACKED_WEIGHTS if packed else 0


def packed_is_bf16_only(case, packed):
    """The packed layout exists for bf16 only: an fp32 workload asking for it
    must be refused on the host (MOE_ERR_UNSUPPORTED) instead of computed."""
    return packed and case.cfg.dtype != "bf16"


def expect_unsupported(fn, *args):
    with pytest.raises(moe.MoeError) as ei:
        fn(*args)
    assert "UNSUPPORTED" in str(ei.value)


@pytest.fixture(scope="module", params=NAMES)
def case(request):
    dev()
    c = Case(request.param)
    yield c
    del c
    torch.cuda.empty_cache()


def test_route(case):
    cfg, p, d = case.cfg, prob(case.cfg), "cuda"
    out = dict(topk_idx=torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=d),
               topk_gate=torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=d),
               counts=torch.empty(cfg.n, dtype=torch.int32, device=d),
               f=torch.empty(cfg.n, dtype=torch.float32, device=d),
               P=torch.empty(cfg.n, dtype=torch.float32, device=d))
    moe.moe_route(p, case.dev["u"], case.dev["centroids"], out["topk_idx"], out["topk_gate"],
                  out["counts"], out["f"], out["P"], workspace(p, d))
    torch.cuda.synchronize()
    ref = case.route
    got = {k: v.cpu().numpy() for k, v in out.items()}
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["f"].view(np.uint32), ref["f"].view(np.uint32))
    eg, ep = elem_rel(got["topk_gate"], ref["topk_gate"]), elem_rel(got["P"], ref["P"])
    tg, tp = gate_tol(cfg.d, cfg.n, case.max_abs_logit), p_tol(cfg.T, cfg.d, cfg.n,
                                                               case.max_abs_logit)
    print(f"{case.name}: gate rel {eg:.2e} (bar {tg:.2e}), P rel {ep:.2e} (bar {tp:.2e})")
    assert eg <= tg
    assert ep <= tp


@pytest.mark.parametrize("alpha", [0.001, 0.1])
def test_balance_loss(case, alpha):
    """The expert-level balance loss alpha * sum_i f_i P_i ("Expert-level
    balance loss") over the oracle's statistics f and P: bit-exact against
    the oracle's plain ascending fp32 sum."""
    cfg, p, d = case.cfg, prob(case.cfg), "cuda"
    f = torch.from_numpy(np.ascontiguousarray(case.route["f"], np.float32)).to(d)
    P = torch.from_numpy(np.ascontiguousarray(case.route["P"], np.float32)).to(d)
    loss = torch.full((4,), float("nan"), dtype=torch.float32, device=d)
    moe.moe_balance_loss(p, f, P, alpha, loss)
    torch.cuda.synchronize()
    got = np.float32(loss[0].item())
    ref = np.float32(oracle.balance_loss(case.route["f"], case.route["P"], alpha))
    assert got.view(np.uint32) == ref.view(np.uint32), (got, ref)


@pytest.mark.parametrize("name", DECODE)
def test_decode_cases_cover_their_paths(name):
    """The few-rows workloads really are few rows per expert, and the skewed
    one has an expert above 32 rows (several passes over its weights)."""
    cfg = ALL[name]
    inp = inputs(name)
    counts = oracle.route(inp["u"], inp["centroids"], cfg.k)["counts"]
    assert cfg.T <= 64 and cfg.T * cfg.k <= 16 * cfg.n
    if cfg.name == "decode_skew_bf16":
        assert counts.max() > 32


@pytest.mark.parametrize("name", EDGE)
def test_edge_cases_exercise_the_rule(name):
    """The tie workloads really put an exact tie at every token's k-th choice
    (k odd, twins adjacent: the lower index is kept, its twin dropped) and
    inside the kept list (a pair in index order); the flat-router workloads
    tie all n experts, so every token keeps 0 .. k-1 with gate 1/n; the
    single-expert workloads give every token gate one."""
    cfg = ALL[name]
    inp = inputs(name)
    r = oracle.route(inp["u"], inp["centroids"], cfg.k)
    idx, gate = r["topk_idx"], r["topk_gate"]
    if cfg.tie_pairs:
        assert cfg.k % 2 == 1
        last = idx[:, cfg.k - 1]
        assert (last % 2 == 0).all()
        assert not (idx[:, :cfg.k - 1] == (last + 1)[:, None]).any()
        assert (idx[:, 1] == idx[:, 0] + 1).all()
    elif cfg.flat_router:
        assert (idx == np.arange(cfg.k)[None, :]).all()
        assert np.allclose(gate, 1.0 / cfg.n, rtol=0, atol=1e-7)
    else:
        assert cfg.n == 1
        assert (idx == 0).all() and (gate == 1.0).all()


@pytest.mark.parametrize("gather", [True, False])
def test_permute(case, gather):
    cfg, p, d = case.cfg, prob(case.cfg), "cuda"
    pm = case.perm
    R = cfg.T * cfg.k
    u = case.dev["u"]
    idx = torch.from_numpy(case.route["topk_idx"]).to(d)
    offsets = torch.empty(cfg.n + 1, dtype=torch.int32, device=d)
    perm = torch.empty(R, dtype=torch.int32, device=d)
    slot = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=d)
    xp = torch.empty((R, cfg.d), dtype=torch_dtype(p), device=d) if gather else None
    moe.moe_permute(p, u, idx, offsets, perm, slot, xp, workspace(p, d))
    torch.cuda.synchronize()
    assert np.array_equal(offsets.cpu().numpy(), pm["offsets"])
    assert np.array_equal(perm.cpu().numpy(), pm["perm_token"])
    assert np.array_equal(slot.cpu().numpy(), pm["slot_of"])
    if gather:
        want = torch.from_numpy(pm["perm_token"].astype(np.int64)).to(d)
        assert torch.equal(xp, u[want])


@pytest.mark.parametrize("packed", [False, True])
def test_grouped_ffn(case, packed):
    """Routed experts: y_perm[slot_of[t, j]] = FFN_{idx[t, j]}(u_t), ungated,
    every slot of every token.  Shared experts (when the workload has them):
    the K_s experts as one dense group of width K_s*d_ff equal the oracle's
    expert-by-expert shared sum."""
    cfg, p, d = case.cfg, prob(case.cfg), "cuda"
    fl = packed_flag(case, packed)
    pm = case.perm
    R = cfg.T * cfg.k
    offs = torch.from_numpy(pm["offsets"]).to(d)
    if packed_is_bf16_only(case, packed):
        expect_unsupported(moe.moe_grouped_ffn, p, cfg.n, R, offs, case.dev["u"],
                           case.dev["w1"], case.dev["w3"], case.dev["w2"], cfg.d_ff, fl,
                           case.dev["u"], workspace(p, d))
        return
    w = case.weights(packed)
    x = case.dev["u"][torch.from_numpy(pm["perm_token"].astype(np.int64)).to(d)].contiguous()
    y = torch.empty((R, cfg.d), dtype=torch_dtype(p), device=d)
    moe.moe_grouped_ffn(p, cfg.n, R, offs, x, w["w1"], w["w3"], w["w2"], cfg.d_ff, fl, y,
                        workspace(p, d))
    torch.cuda.synchronize()
    rows = torch.from_numpy(pm["slot_of"][case.toks].ravel().astype(np.int64)).to(d)
    got = host(y[rows]).reshape(len(case.toks), cfg.k, cfg.d)
    want = case.layer["Y"]
    # every slot position separately, not only the largest outputs
    for j in range(cfg.k):
        assert rel(got[:, j], want[:, j]) <= exact_tol(cfg), j
    if cfg.K_s == 0:
        return
    s_out = torch.empty((cfg.T, cfg.d), dtype=torch_dtype(p), device=d)
    offs1 = torch.tensor([0, cfg.T], dtype=torch.int32, device=d)
    moe.moe_grouped_ffn(p, 1, cfg.T, offs1, case.dev["u"], w["ws1"], w["ws3"], w["ws2"],
                        cfg.K_s * cfg.d_ff, fl, s_out, workspace(p, d))
    torch.cuda.synchronize()
    got = host(s_out[torch.from_numpy(case.toks).to(d)])
    assert rel(got, case.layer["S"]) <= exact_tol(cfg)


def test_pack_layout(case):
    """moe_pack_weights places element (r, k) of a [rows][K] matrix at
    band r/32, block k/16, offset ((r%32) + 32*((k%16)/8))*8 + k%8 (bf16;
    fp32 weights are refused)."""
    cfg = case.cfg
    if cfg.dtype != "bf16":
        t = case.dev["w2"]
        expect_unsupported(moe.moe_pack_weights, prob(cfg), t.numel() // t.shape[-1],
                           t.shape[-1], t, torch.empty_like(t))
        return
    src = case.inp["w2"]
    rows, K = src.shape[0] * src.shape[1], src.shape[2]
    a = src.reshape(rows, K)
    want = (a.reshape(rows // 32, 32, K // 16, 2, 8)      # band, r, kb, h, e
             .transpose(0, 2, 3, 1, 4)                     # band, kb, h, r, e
             .reshape(-1))
    got = case.weights(True)["w2"].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("terms", ["all", "no_residual", "experts_only"])
def test_combine(case, terms):
    """Combine on seeded random expert outputs against the oracle's combine."""
    cfg, p, d = case.cfg, prob(case.cfg), "cuda"
    rng = np.random.default_rng(123)
    R = cfg.T * cfg.k
    yp = rng.standard_normal((R, cfg.d), dtype=np.float32)
    sh = rng.standard_normal((cfg.T, cfg.d), dtype=np.float32)
    if cfg.dtype == "bf16":
        yp = moe_synth.f32_to_bf16_bits(yp)
        sh = moe_synth.f32_to_bf16_bits(sh)
    res = case.inp["u"] if terms == "all" else None
    shared = sh if terms != "experts_only" else None
    want = oracle.combine(yp, case.perm["slot_of"], case.route["topk_gate"], shared, res)
    h = torch.empty((cfg.T, cfg.d), dtype=torch_dtype(p), device=d)
    moe.moe_combine(p, case.dev["u"] if terms == "all" else None, to_device(shared, d),
                    to_device(yp, d), torch.from_numpy(case.perm["slot_of"]).to(d),
                    torch.from_numpy(case.route["topk_gate"]).to(d), h)
    torch.cuda.synchronize()
    # one rounding of the fp32 sum to the storage type
    tol = 1e-5 if cfg.dtype == "f32" else 2.0 ** -8
    assert rel(host(h), want) <= tol


def run_layer(case, flags=0, ws=None):
    cfg, p, d = case.cfg, prob(case.cfg), "cuda"
    t = case.weights(bool(flags & moe.MOE_PACKED_WEIGHTS))
    h = torch.empty((cfg.T, cfg.d), dtype=torch_dtype(p), device=d)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=d)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=d)
    counts = torch.empty(cfg.n, dtype=torch.int32, device=d)
    f = torch.empty(cfg.n, dtype=torch.float32, device=d)
    P = torch.empty(cfg.n, dtype=torch.float32, device=d)
    ws = workspace(p, d) if ws is None else ws
    moe.moe_layer_fwd(p, t["u"], t["centroids"], t["w1"], t["w3"], t["w2"], t["ws1"], t["ws3"],
                      t["ws2"], h, idx, gate, counts, f, P, flags, ws)
    torch.cuda.synchronize()
    return dict(h=h, topk_idx=idx, topk_gate=gate, counts=counts, f=f, P=P)


@pytest.mark.parametrize("packed", [False, True])
def test_layer(case, packed):
    cfg = case.cfg
    if packed_is_bf16_only(case, packed):
        expect_unsupported(run_layer, case, packed_flag(case, packed))
        return
    out = run_layer(case, packed_flag(case, packed))
    o = case.layer
    assert np.array_equal(out["topk_idx"].cpu().numpy(), o["topk_idx"])
    assert np.array_equal(out["counts"].cpu().numpy(), o["counts"])
    assert np.array_equal(out["f"].cpu().numpy().view(np.uint32), o["f"].view(np.uint32))
    lmax = case.max_abs_logit
    assert elem_rel(out["topk_gate"].cpu().numpy(), o["topk_gate"]) <= gate_tol(cfg.d, cfg.n, lmax)
    assert elem_rel(out["P"].cpu().numpy(), o["P"]) <= p_tol(cfg.T, cfg.d, cfg.n, lmax)
    got = host(out["h"][torch.from_numpy(case.toks).to("cuda")])
    assert rel(got, o["h"]) <= exact_tol(cfg)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("flags", ["no_residual", "no_shared_no_residual"])
def test_layer_components(case, flags, packed):
    """The residual u and the shared experts dominate |h|; dropping them checks
    the routed sum and the shared sum at their own scale."""
    cfg = case.cfg
    fl = moe.MOE_NO_RESIDUAL | (moe.MOE_NO_SHARED if flags == "no_shared_no_residual" else 0)
    if packed_is_bf16_only(case, packed):
        expect_unsupported(run_layer, case, fl | packed_flag(case, packed))
        return
    out = run_layer(case, fl | packed_flag(case, packed))
    o = case.layer
    want = o["ysum"] if flags == "no_residual" else o["ysum"] - o["S"]
    got = host(out["h"][torch.from_numpy(case.toks).to("cuda")])
    assert rel(got, want) <= exact_tol(cfg)


def test_layer_bitwise_deterministic(case):
    """Two runs (the second on a workspace filled with junk) give identical bits."""
    fl = moe.MOE_PACKED_WEIGHTS if case.cfg.dtype == "bf16" else 0
    a = run_layer(case, fl)
    ws = workspace(prob(case.cfg), "cuda")
    ws.fill_(0xA5)
    b = run_layer(case, fl, ws=ws)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_layer_graph_replays(case):
    """The layer captured as a HIP graph reproduces the eager bits on every
    replay, back to back and after an eager call on the same workspace, with
    junk written to the outputs before each replay."""
    cfg = case.cfg
    fl = moe.MOE_PACKED_WEIGHTS if cfg.dtype == "bf16" else 0
    want = run_layer(case, fl)
    p, d = prob(cfg), "cuda"
    t = case.weights(bool(fl & moe.MOE_PACKED_WEIGHTS))
    out = {k: torch.empty_like(v) for k, v in want.items()}
    ws = workspace(p, d)
    args = lambda: (p, t["u"], t["centroids"], t["w1"], t["w3"], t["w2"], t["ws1"], t["ws3"],
                    t["ws2"], out["h"], out["topk_idx"], out["topk_gate"], out["counts"],
                    out["f"], out["P"], fl, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layer_fwd(*args())  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_fwd(*args())
    for i, eager_between in enumerate((False, True, False)):
        for v in out.values():
            v.fill_(-3)
        if eager_between:
            run_layer(case, fl, ws=ws)
        g.replay()
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(out[k], want[k]), (i, k)
