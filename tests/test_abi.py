"""C ABI checks that need no GPU: the library loads, exports every entry point
include/moe.h declares, and rejects bad arguments on the host before any HIP
call (fake, never-dereferenced addresses are enough for that)."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_layer_34_amd as moe
from mixture_experts_layer_34_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

A = 0x100000          # aligned fake device address
MIS = 0x100001        # misaligned fake device address
BIG = 1 << 40         # fake workspace size

S = {v: k for k, v in _native.STATUS_NAMES.items()}


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_fwd",
                 "moe_workspace_bytes", "moe_status_str"):
        assert want in names


# Section titles of the DeepSeekMoE explainer (deepforge.srivtx.xyz) that
# define what the boundary's compute entry points do.
PAGE_SECTIONS = ("Routing in a classic MoE layer", "Top-k routing, from affinities to gates",
                 "Expert-level balance loss", "What the 16B configuration looks like")
BOUNDARY = ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_fwd",
            "moe_balance_loss")


def declaration_comment(name):
    """The comment block right before the declaration of `name`."""
    txt = open(HEADER).read()
    at = re.search(r"\n(moe_status|size_t|int|const char \*)\s*" + name + r"\s*\(", txt)
    assert at, name
    head = txt[:at.start()]
    end = head.rstrip().rfind("*/")
    start = head.rfind("/*", 0, end)
    assert end > 0 and start >= 0 and not head[end + 2:].strip(), name
    return " ".join(head[start:end].replace("*", " ").split())


@pytest.mark.parametrize("name", BOUNDARY)
def test_boundary_declarations_cite_the_pages(name):
    """Every compute entry point of the boundary names the page section that
    defines its operation."""
    block = declaration_comment(name)
    assert any(f'"{sec}"' in block for sec in PAGE_SECTIONS), (name, block[:200])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_native.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(moe_\w+)", out))
    assert set(declared_functions()) <= exported


def p16(**kw):
    base = dict(T=4096, d=2048, N=16, m=4, K=2, K_s=2, d_ff=1408, dtype="bf16")
    base.update(kw)
    return moe.problem(**base)


def status(fn, *args):
    with pytest.raises(moe.MoeError) as ei:
        fn(*args)
    return _native.STATUS_NAMES[ei.value.status]


def test_status_strings():
    for code in range(8):
        assert moe.moe_status_str(code)
    assert moe.moe_status_str(99) == "unknown status"


def test_last_hip_error_starts_clear():
    # host-side validation failures never touch the HIP error slot
    p = p16(T=0)
    assert status(moe.moe_route, p, A, A, A, A, A, A, A, A, BIG) == "MOE_ERR_SHAPE"
    code, text = moe.moe_last_hip_error()
    assert code == 0 and text


@pytest.mark.parametrize("kw,why", [
    (dict(T=0), "T < 1"),
    (dict(d=48), "d not a multiple of 32"),
    (dict(d=0), "d < 32"),
    (dict(d_ff=100), "d_ff not a multiple of 32"),
    (dict(N=0), "N < 1"),
    (dict(m=0), "m < 1"),
    (dict(K_s=-1), "K_s < 0"),
    (dict(K=1, K_s=4), "k < 1"),
    (dict(N=2, m=1, K=3, K_s=0), "k > n"),
    (dict(N=257, m=1, K=1, K_s=0), "n > 256"),
    (dict(N=128, m=1, K=65, K_s=0), "k > 64"),
    (dict(T=1 << 29, N=64, m=1, K=8, K_s=0), "T*k overflows int32"),
    (dict(T=1 << 17, d=4096), "T*k*d reaches 2^31 elements"),
    (dict(T=1 << 18, d=64, d_ff=1408), "T*k*d_ff reaches 2^31 elements"),
    (dict(T=1, d=65536, d_ff=32768, K_s=0, K=1, m=1, N=1), "d*d_ff reaches 2^31 elements"),
    (dict(T=1, d=32768, d_ff=16384, K_s=4, K=5, m=1, N=1), "K_s*d_ff*d reaches 2^31"),
])
def test_shape_validation(kw, why):
    p = p16(**kw)
    assert moe.moe_workspace_bytes(p) == 0, why
    assert status(moe.moe_route, p, A, A, A, A, A, A, A, A, BIG) == "MOE_ERR_SHAPE", why
    assert status(moe.moe_layer_fwd, p, A, A, A, A, A, A, A, A, A, A, A, A, A, A, 0, A,
                  BIG) == "MOE_ERR_SHAPE", why


def test_dtype_validation():
    p = p16()
    p.dtype = 7
    assert moe.moe_workspace_bytes(p) == 0
    assert status(moe.moe_combine, p, A, A, A, A, A, A) == "MOE_ERR_DTYPE"


def test_null_problem():
    r = _native.lib.moe_route(None, A, A, A, A, A, A, A, A, BIG, None)
    assert _native.STATUS_NAMES[r] == "MOE_ERR_NULL"
    assert _native.lib.moe_workspace_bytes(None) == 0


def test_route_pointer_checks():
    p = p16()
    ws = moe.moe_workspace_bytes(p)
    for i in range(7):
        args = [A] * 7
        args[i] = None
        assert status(moe.moe_route, p, *args, A, ws) == "MOE_ERR_NULL", i
        args[i] = MIS
        assert status(moe.moe_route, p, *args, A, ws) == "MOE_ERR_ALIGN", i
    assert status(moe.moe_route, p, *[A] * 7, None, ws) == "MOE_ERR_WORKSPACE"
    assert status(moe.moe_route, p, *[A] * 7, A, ws - 1) == "MOE_ERR_WORKSPACE"
    assert status(moe.moe_route, p, *[A] * 7, MIS, ws) == "MOE_ERR_ALIGN"


def test_permute_pointer_checks():
    p = p16()
    ws = moe.moe_workspace_bytes(p)
    # u may be NULL only when x_perm is NULL
    assert status(moe.moe_permute, p, None, A, A, A, A, A, A, ws) == "MOE_ERR_NULL"
    for i in (1, 2, 3, 4):
        args = [A] * 6
        args[i] = None
        assert status(moe.moe_permute, p, *args, A, ws) == "MOE_ERR_NULL", i
        args[i] = MIS
        assert status(moe.moe_permute, p, *args, A, ws) == "MOE_ERR_ALIGN", i
    assert status(moe.moe_permute, p, A, A, A, A, A, MIS, A, ws) == "MOE_ERR_ALIGN"
    assert status(moe.moe_permute, p, A, A, A, A, A, A, A, 16) == "MOE_ERR_WORKSPACE"


def test_grouped_ffn_checks():
    p = p16()
    ws = moe.moe_workspace_bytes(p)
    R = p.T * 6
    ok = [A] * 5
    st = moe.moe_grouped_ffn
    assert status(st, p, 0, R, *ok, 1408, 0, A, A, ws) == "MOE_ERR_SHAPE"
    assert status(st, p, 257, R, *ok, 1408, 0, A, A, ws) == "MOE_ERR_SHAPE"
    assert status(st, p, 64, 0, *ok, 1408, 0, A, A, ws) == "MOE_ERR_SHAPE"
    assert status(st, p, 64, R, *ok, 1400, 0, A, A, ws) == "MOE_ERR_SHAPE"
    assert status(st, p, 64, R, *ok, 1408, 8, A, A, ws) == "MOE_ERR_SHAPE"   # unknown flag
    assert status(st, p, 1, R, *ok, 1 << 20, 0, A, A, ws) == "MOE_ERR_SHAPE"  # d_ff_group*d
    assert status(st, p, 64, R + 1, *ok, 1408, 0, A, A, ws) == "MOE_ERR_WORKSPACE"
    assert status(st, p, 64, R, *ok, 1408 * 8, 0, A, A, ws) == "MOE_ERR_WORKSPACE"
    for i in range(5):
        args = [A] * 5
        args[i] = None
        assert status(st, p, 64, R, *args, 1408, 0, A, A, ws) == "MOE_ERR_NULL"
        args[i] = MIS
        assert status(st, p, 64, R, *args, 1408, 0, A, A, ws) == "MOE_ERR_ALIGN"
    assert status(st, p, 64, R, *ok, 1408, 0, None, A, ws) == "MOE_ERR_NULL"
    pf = p16(dtype="f32")
    assert status(st, pf, 64, R, *ok, 1408, moe.MOE_PACKED_WEIGHTS, A, A,
                  moe.moe_workspace_bytes(pf)) == "MOE_ERR_UNSUPPORTED"


def test_pack_weights_checks():
    p = p16()
    pk = moe.moe_pack_weights
    assert status(pk, p16(dtype="f32"), 64, 64, A, A + (1 << 20)) == "MOE_ERR_UNSUPPORTED"
    assert status(pk, p, 48, 64, A, A + (1 << 20)) == "MOE_ERR_SHAPE"     # rows % 32
    assert status(pk, p, 64, 48, A, A + (1 << 20)) == "MOE_ERR_SHAPE"     # K % 32
    assert status(pk, p, 64, 64, A, A + 4096) == "MOE_ERR_SHAPE"          # overlap
    assert status(pk, p, 64, 64, None, A) == "MOE_ERR_NULL"
    assert status(pk, p, 64, 64, MIS, A + (1 << 20)) == "MOE_ERR_ALIGN"
    bad = p16(T=0)
    assert status(pk, bad, 64, 64, A, A + (1 << 20)) == "MOE_ERR_SHAPE"


def test_combine_checks():
    p = p16()
    for i in range(4):
        args = [A] * 4
        args[i] = None
        assert status(moe.moe_combine, p, A, A, *args) == "MOE_ERR_NULL", i
        args[i] = MIS
        assert status(moe.moe_combine, p, A, A, *args) == "MOE_ERR_ALIGN", i
    assert status(moe.moe_combine, p, MIS, None, A, A, A, A) == "MOE_ERR_ALIGN"
    assert status(moe.moe_combine, p, None, MIS, A, A, A, A) == "MOE_ERR_ALIGN"


def test_balance_loss_checks():
    p = p16()
    for i in range(3):
        args = [A] * 3
        args[i] = None
        assert status(moe.moe_balance_loss, p, args[0], args[1], 0.01, args[2]) == \
            "MOE_ERR_NULL", i
        args[i] = MIS
        assert status(moe.moe_balance_loss, p, args[0], args[1], 0.01, args[2]) == \
            "MOE_ERR_ALIGN", i
    assert status(moe.moe_balance_loss, p16(T=0), A, A, 0.01, A) == "MOE_ERR_SHAPE"


def test_layer_fwd_checks():
    p = p16()
    ws = moe.moe_workspace_bytes(p)
    full = [A] * 14
    # bad flag bits
    assert status(moe.moe_layer_fwd, p, *full, 16, A, ws) == "MOE_ERR_SHAPE"
    pf = p16(dtype="f32")
    for fl in (moe.MOE_PACKED_WEIGHTS, moe.MOE_SAVE_FOR_BACKWARD):
        assert status(moe.moe_layer_fwd, pf, *full, fl, A,
                      moe.moe_workspace_bytes(pf)) == "MOE_ERR_UNSUPPORTED"
    # keeping the pre-activations needs the larger workspace
    wt = moe.moe_train_workspace_bytes(p)
    assert wt > ws and wt % 256 == 0 and moe.moe_train_workspace_bytes(pf) == 0
    assert status(moe.moe_layer_fwd, p, *full, moe.MOE_SAVE_FOR_BACKWARD, A,
                  ws) == "MOE_ERR_WORKSPACE"
    # shared weights required when K_s > 0 ...
    args = list(full)
    args[5] = None
    assert status(moe.moe_layer_fwd, p, *args, 0, A, ws) == "MOE_ERR_NULL"
    # ... and misaligned ones rejected
    args[5] = MIS
    assert status(moe.moe_layer_fwd, p, *args, 0, A, ws) == "MOE_ERR_ALIGN"
    for i in (0, 1, 2, 3, 4, 8, 9, 10, 11, 12, 13):
        args = list(full)
        args[i] = None
        assert status(moe.moe_layer_fwd, p, *args, 0, A, ws) == "MOE_ERR_NULL", i
        args[i] = MIS
        assert status(moe.moe_layer_fwd, p, *args, 0, A, ws) == "MOE_ERR_ALIGN", i
    assert status(moe.moe_layer_fwd, p, *full, 0, A, ws - 256) == "MOE_ERR_WORKSPACE"


def test_noalloc_checks():
    """moe_layer_fwd_noalloc refuses, on the host, problems whose workspace
    exceeds its fixed scratch and the flag whose workspace the backward would
    need to name; bad shapes as moe_layer_fwd."""
    full = [A] * 14
    assert status(moe.moe_layer_fwd_noalloc, p16(), *full, 0) == "MOE_ERR_WORKSPACE"
    small = p16(T=64)
    assert moe.moe_workspace_bytes(small) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    assert status(moe.moe_layer_fwd_noalloc, small, *full, moe.MOE_SAVE_FOR_BACKWARD) == \
        "MOE_ERR_UNSUPPORTED"
    assert status(moe.moe_layer_fwd_noalloc, p16(T=0), *full, 0) == "MOE_ERR_SHAPE"


def test_workspace_grows_with_problem():
    a = moe.moe_workspace_bytes(p16())
    b = moe.moe_workspace_bytes(p16(T=8192))
    assert 0 < a < b
    assert a % 256 == 0


def test_one_hip_runtime_per_process():
    # The binding loads torch's HIP runtime before libmoe.so, so the process
    # maps exactly one libamdhip64 whichever module was imported first.
    code = ("import mixture_experts_layer_34_amd as m; m.moe_status_str(0); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout
    assert out.count("libamdhip64") == 1, out


def test_layer_kernel_sequence():
    # Batches of at most 64 bf16 tokens: logits spread over the GPU, then one
    # workgroup routes and groups the batch.  Larger batches: per-block
    # routing, then the one-pass grouping kernel for histogram tables of up
    # to 32768 entries, the separate scan and scatter beyond.
    assert moe.moe_layer_kernels(p16(T=64)) == ["logits", "route_group", "up_swiglu", "down",
                                                "combine"]
    assert moe.moe_layer_kernels(p16(T=64, dtype="f32"))[:2] == ["route", "group"]
    assert moe.moe_layer_kernels(p16(T=65))[:2] == ["route", "group"]
    assert moe.moe_layer_kernels(p16(T=8192))[:2] == ["route", "group"]
    assert moe.moe_layer_kernels(p16(T=8208))[:3] == ["route", "scan", "scatter"]
    assert moe.moe_layer_kernels(p16(dtype="f32"))[2:4] == ["up_swiglu_f32", "down_f32"]


def test_layer_bwd_checks():
    p = p16()
    ws = moe.moe_bwd_workspace_bytes(p)
    assert ws > 0 and ws % 256 == 0
    assert moe.moe_bwd_workspace_bytes(p16(dtype="f32")) == 0
    # u, centroids, w1, w3, w2, ws1, ws3, ws2, topk_idx, topk_gate, f, fwd_ws, dh
    ins = [A] * 11 + [None, A]
    # du, dcent, dw1, dw3, dw2, dws1, dws3, dws2
    outs = [A] * 8
    call = lambda pp, i, a, o, flags, w: moe.moe_layer_bwd(pp, *i, a, *o, flags, A, w)
    assert status(call, p16(dtype="f32"), ins, 0.0, outs, 0, BIG) == "MOE_ERR_UNSUPPORTED"
    # packed weights are accepted: the same checks apply
    assert status(call, p, ins, 0.0, outs, moe.MOE_PACKED_WEIGHTS, 0) == "MOE_ERR_WORKSPACE"
    assert status(call, p, ins, 0.0, outs, 16, BIG) == "MOE_ERR_SHAPE"
    assert status(call, p16(T=0), ins, 0.0, outs, 0, BIG) == "MOE_ERR_SHAPE"
    # the forward's kept workspace: given exactly when the flag says so
    sv = moe.MOE_SAVE_FOR_BACKWARD
    with_fw = ins[:11] + [A, A]
    assert status(call, p, ins, 0.0, outs, sv, BIG) == "MOE_ERR_NULL"
    assert status(call, p, with_fw, 0.0, outs, 0, BIG) == "MOE_ERR_SHAPE"
    assert status(call, p, ins[:11] + [MIS, A], 0.0, outs, sv, BIG) == "MOE_ERR_ALIGN"
    assert status(call, p, with_fw, 0.0, outs, sv, 0) == "MOE_ERR_WORKSPACE"
    for i in range(13):
        if i in (5, 6, 7, 11):
            continue  # shared weights: checked below; fwd_ws: above
        bad = list(ins)
        bad[i] = None
        assert status(call, p, bad, 0.0, outs, 0, BIG) == "MOE_ERR_NULL", i
        bad[i] = MIS
        assert status(call, p, bad, 0.0, outs, 0, BIG) == "MOE_ERR_ALIGN", i
    for i in range(8):
        bad = list(outs)
        bad[i] = None
        assert status(call, p, ins, 0.0, bad, 0, BIG) == "MOE_ERR_NULL", i
    # shared experts' weights and gradients may be NULL when they are dropped
    no_sh_in = ins[:5] + [None] * 3 + ins[8:]
    no_sh_out = outs[:5] + [None] * 3
    assert status(call, p, no_sh_in, 0.0, outs, 0, BIG) == "MOE_ERR_NULL"
    assert status(call, p, ins, 0.0, no_sh_out, 0, BIG) == "MOE_ERR_NULL"
    assert status(call, p, no_sh_in, 0.0, no_sh_out, moe.MOE_NO_SHARED, ws - 256) == \
        "MOE_ERR_WORKSPACE"
    assert status(call, p, ins, 0.0, outs, 0, 0) == "MOE_ERR_WORKSPACE"


@pytest.mark.parametrize("kw,why", [
    # T * ceil8(n) reaches 2^31: the bf16 softmax gradient's byte offsets
    (dict(T=(1 << 31) // 64, d=32, d_ff=32, N=64, m=1, K=1, K_s=0), "T*ldl"),
    # one expert's fp32 weight gradient reaches 2^31 - 16 bytes
    (dict(T=64, d=16384, d_ff=32768, K_s=0), "d_ff*d*4"),
    # the shared experts' fp32 weight gradient does
    (dict(T=64, d=8192, d_ff=16384, K=2, K_s=4, m=4), "K_s*d_ff*d*4"),
])
def test_layer_bwd_rejects_sizes_its_offsets_cannot_reach(kw, why):
    """Bounds of the backward's 32-bit addressing are checked on the host,
    before anything is enqueued (MOE_ERR_SHAPE), not at a later launch."""
    p = p16(**kw)
    assert moe.moe_workspace_bytes(p) > 0, why  # a valid forward problem
    ins = [A] * 11 + [None, A]
    outs = [A] * 8
    assert status(lambda: moe.moe_layer_bwd(p, *ins, 0.0, *outs, 0, A, BIG)) == \
        "MOE_ERR_SHAPE", why
    assert moe.moe_bwd_workspace_bytes(p) > 0, why


def test_layer_bwd_kernel_sequence():
    assert moe.moe_layer_bwd_kernels(p16()) == [
        "hist", "scan", "scatter", "gather", "logits", "q", "ab_swiglu", "dx", "softmax_bwd",
        "du", "wgrad", "dcent_sum"]
    # after a forward that kept its grouping and pre-activations
    assert moe.moe_layer_bwd_kernels(p16(), moe.MOE_SAVE_FOR_BACKWARD) == [
        "gather", "q", "swiglu_bwd", "dx", "softmax_bwd", "du", "wgrad", "dcent_sum"]
