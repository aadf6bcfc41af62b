"""Builds libmoe.so (HIP for gfx950) in the package directory.

    python -m mixture_experts_layer_34_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "moe")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["abi.hip", "route.hip", "permute.hip", "gemm.hip", "skinny.hip", "bwd.hip"]
ARCH = "gfx950"
# Per-file flags.  bwd.hip: no wave-level combining of atomics (it would
# wait for an atomic's reply where it is issued; the weight-gradient kernel
# takes its reply much later, under a wait it has anyway).
EXTRA = {"bwd.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (device
# code is built as usual): for CPU tests of the argument validation, with the
# compiler's ASan runtime preloaded (host_sanitizer_runtime()).
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def host_sanitizer_runtime() -> str:
    """Path of the ASan runtime (with the UBSan handlers) hipcc's host
    compiler links against; preload it to load a host-sanitized libmoe.so."""
    r = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def _compile(src: str, obj: str = OBJ, extra=()) -> str:
    out = os.path.join(obj, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + flags() + EXTRA.get(src, []) + list(extra) +
           ["-c", os.path.join(CSRC, src), "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, lib: str = LIB, sanitize_host: bool = False) -> str:
    obj = OBJ + ("_host_san" if sanitize_host else "")
    extra = HOST_SAN if sanitize_host else []
    os.makedirs(obj, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + list(extra) + \
        ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
