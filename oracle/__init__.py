"""ctypes wrapper of the plain-C CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU path.  The arithmetic lives in
moe_oracle.c; this file only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test of the pins themselves may point this at a deliberately broken build.
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

F32, BF16 = 0, 1
_lib = None


def build() -> str:
    subprocess.run(["make", "-s", "-C", _HERE, "liboracle.so"], check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_sizes.argtypes = [i32, i32, i32, i32, P, P]
    lib.oracle_route.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
    lib.oracle_balance_loss.argtypes = [i32, P, P, ctypes.c_float]
    lib.oracle_balance_loss.restype = ctypes.c_float
    lib.oracle_permute.argtypes = [i64, i32, i32, P, P, P, P]
    lib.oracle_expert.argtypes = [i32, i32, i32, i32, P, P, P, P, P]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_layer_bwd.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32,
                                     P, P, P, P, P, P, P, P,
                                     P, P, P, ctypes.c_double, i32, P, i64, P, P,
                                     P, i32, P, P, P, P, P, P]
    lib.oracle_combine.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_layer.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32,
                                 P, P, P, P, P, P, P, P, P, i64,
                                 P, P, P, P, P, P, P, P, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def sizes(N: int, m: int, K: int, K_s: int) -> tuple[int, int]:
    n, k = ctypes.c_int(), ctypes.c_int()
    rc = _load().oracle_sizes(N, m, K, K_s, ctypes.byref(n), ctypes.byref(k))
    if rc != 0:
        raise ValueError(f"invalid (N, m, K, K_s) = {(N, m, K, K_s)}")
    return n.value, k.value


def route(u: np.ndarray, centroids: np.ndarray, k: int, want_scores: bool = False) -> dict:
    u, centroids = _c(u), _c(centroids)
    T, d = u.shape
    n = centroids.shape[0]
    dt = _dt(u)
    assert _dt(centroids) == dt and centroids.shape[1] == d
    out = dict(topk_idx=np.empty((T, k), np.int32), topk_gate=np.empty((T, k), np.float32),
               counts=np.empty(n, np.int32), f=np.empty(n, np.float32),
               P=np.empty(n, np.float32))
    if want_scores:
        out["logits"] = np.empty((T, n), np.float32)
        out["scores"] = np.empty((T, n), np.float32)
    rc = _load().oracle_route(T, d, n, k, dt, _p(u), _p(centroids), _p(out["topk_idx"]),
                              _p(out["topk_gate"]), _p(out.get("logits")),
                              _p(out.get("scores")), _p(out["counts"]), _p(out["f"]),
                              _p(out["P"]))
    if rc != 0:
        raise RuntimeError(f"oracle_route failed ({rc})")
    return out


def balance_loss(f: np.ndarray, P: np.ndarray, alpha: float) -> float:
    f = np.ascontiguousarray(f, np.float32)
    P = np.ascontiguousarray(P, np.float32)
    return float(_load().oracle_balance_loss(f.size, _p(f), _p(P), alpha))


def permute(topk_idx: np.ndarray, n: int) -> dict:
    idx = np.ascontiguousarray(topk_idx, np.int32)
    T, k = idx.shape
    out = dict(offsets=np.empty(n + 1, np.int32), perm_token=np.empty(T * k, np.int32),
               slot_of=np.empty((T, k), np.int32))
    rc = _load().oracle_permute(T, n, k, _p(idx), _p(out["offsets"]), _p(out["perm_token"]),
                                _p(out["slot_of"]))
    if rc != 0:
        raise RuntimeError(f"oracle_permute failed ({rc})")
    return out


def expert(x: np.ndarray, e: int, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Routed expert e of w1/w3 [n][d_ff][d], w2 [n][d][d_ff] on one fp32 vector."""
    x = np.ascontiguousarray(x, np.float32)
    w1, w3, w2 = _c(w1), _c(w3), _c(w2)
    n, d_ff, d = w1.shape
    assert x.shape == (d,) and 0 <= e < n
    y = np.empty(d, np.float32)
    rc = _load().oracle_expert(d, d_ff, e, _dt(w1), _p(x), _p(w1), _p(w3), _p(w2), _p(y))
    if rc != 0:
        raise RuntimeError(f"oracle_expert failed ({rc})")
    return y


def layer(inp: dict, N: int, m: int, K: int, K_s: int, toks=None) -> dict:
    """Whole layer.  inp holds u, centroids, w1, w3, w2, ws1, ws3, ws2 (storage
    type arrays, see moe_synth.make_inputs).  toks: token subset for the expert
    sums (all tokens when None)."""
    u = _c(inp["u"])
    T, d = u.shape
    dt = _dt(u)
    w1 = _c(inp["w1"])
    d_ff = w1.shape[1]
    n, k = sizes(N, m, K, K_s)
    assert w1.shape[0] == n
    if toks is None:
        tk = None
        nt = T
    else:
        tk = np.ascontiguousarray(toks, np.int64)
        nt = tk.size
    out = dict(topk_idx=np.empty((T, k), np.int32), topk_gate=np.empty((T, k), np.float32),
               counts=np.empty(n, np.int32), f=np.empty(n, np.float32),
               P=np.empty(n, np.float32), Y=np.empty((nt, k, d), np.float32),
               S=np.empty((nt, d), np.float32), ysum=np.empty((nt, d), np.float32),
               h=np.empty((nt, d), np.float32))
    ws = [(_c(inp.get(x)) if K_s > 0 else None) for x in ("ws1", "ws3", "ws2")]
    rc = _load().oracle_layer(T, d, N, m, K, K_s, d_ff, dt, _p(u), _p(_c(inp["centroids"])),
                              _p(w1), _p(_c(inp["w3"])), _p(_c(inp["w2"])),
                              _p(ws[0]), _p(ws[1]), _p(ws[2]), _p(tk), nt,
                              _p(out["topk_idx"]), _p(out["topk_gate"]), _p(out["counts"]),
                              _p(out["f"]), _p(out["P"]), _p(out["Y"]), _p(out["S"]),
                              _p(out["ysum"]), _p(out["h"]))
    if rc != 0:
        raise RuntimeError(f"oracle_layer failed ({rc})")
    return out


def combine(y_perm: np.ndarray, slot_of: np.ndarray, gate: np.ndarray, shared=None,
            residual=None) -> np.ndarray:
    """h = sum_j gate * y_perm[slot_of] + shared + residual (fp32 result)."""
    y_perm = _c(y_perm)
    slot_of = np.ascontiguousarray(slot_of, np.int32)
    gate = np.ascontiguousarray(gate, np.float32)
    T, k = slot_of.shape
    d = y_perm.shape[1]
    dt = _dt(y_perm)
    for a in (shared, residual):
        assert a is None or (_dt(a) == dt and a.shape == (T, d))
    h = np.empty((T, d), np.float32)
    rc = _load().oracle_combine(T, d, k, dt, _p(_c(residual)), _p(_c(shared)), _p(y_perm),
                                _p(slot_of), _p(gate), _p(h))
    if rc != 0:
        raise RuntimeError(f"oracle_combine failed ({rc})")
    return h


BWD_NO_RESIDUAL, BWD_NO_SHARED = 1, 2


def layer_bwd(inp: dict, N: int, m: int, K: int, K_s: int, topk_idx: np.ndarray, f: np.ndarray,
              dh: np.ndarray, alpha: float, flags: int = 0, toks=None, want_dcent: bool = True,
              experts=None, want_shared: bool = True) -> dict:
    """Gradients of sum <dh, h> + alpha * sum_i f_i P_i (fp64 results).
    topk_idx and f are the routing of the forward (oracle.route).  toks:
    token rows of du (all tokens when None); experts: routed experts whose
    weight gradients are formed (none when None)."""
    u = _c(inp["u"])
    T, d = u.shape
    dt = _dt(u)
    w1 = _c(inp["w1"])
    d_ff = w1.shape[1]
    n, k = sizes(N, m, K, K_s)
    assert w1.shape[0] == n and topk_idx.shape == (T, k) and dh.shape == (T, d)
    tk = None if toks is None else np.ascontiguousarray(toks, np.int64)
    nt = T if tk is None else tk.size
    ex = None if experts is None else np.ascontiguousarray(experts, np.int32)
    ne = 0 if ex is None else ex.size
    shared = K_s > 0 and not (flags & BWD_NO_SHARED)
    out = dict(du=np.empty((nt, d), np.float64))
    if want_dcent:
        out["dcent"] = np.empty((n, d), np.float64)
    if ne:
        out["dw1"] = np.empty((ne, d_ff, d), np.float64)
        out["dw3"] = np.empty((ne, d_ff, d), np.float64)
        out["dw2"] = np.empty((ne, d, d_ff), np.float64)
    if shared and want_shared:
        out["dws1"] = np.empty((K_s * d_ff, d), np.float64)
        out["dws3"] = np.empty((K_s * d_ff, d), np.float64)
        out["dws2"] = np.empty((d, K_s * d_ff), np.float64)
    ws = [(_c(inp.get(x)) if K_s > 0 else None) for x in ("ws1", "ws3", "ws2")]
    rc = _load().oracle_layer_bwd(
        T, d, N, m, K, K_s, d_ff, dt, _p(u), _p(_c(inp["centroids"])), _p(w1),
        _p(_c(inp["w3"])), _p(_c(inp["w2"])), _p(ws[0]), _p(ws[1]), _p(ws[2]),
        _p(np.ascontiguousarray(topk_idx, np.int32)), _p(np.ascontiguousarray(f, np.float32)),
        _p(np.ascontiguousarray(dh, np.float32)), float(alpha), flags, _p(tk), nt,
        _p(out["du"]), _p(out.get("dcent")), _p(ex), ne, _p(out.get("dw1")),
        _p(out.get("dw3")), _p(out.get("dw2")), _p(out.get("dws1")), _p(out.get("dws3")),
        _p(out.get("dws2")))
    if rc != 0:
        raise RuntimeError(f"oracle_layer_bwd failed ({rc})")
    return out


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().oracle_threads())
