"""Build libpagedkv.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_kv_cache_45_amd.build          # or build() from Python

Each translation unit is compiled to an object in parallel, then linked.  Floating
point is compiled without fast-math (correctly rounded fp32 division is needed for
bit-exact quantisation) and with the packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpagedkv.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.cpp", "pack3.hip", "append.hip", "slots.hip", "decode.hip",
           "decode_same_d128.hip", "decode_u3_d128.hip", "decode_fp8_d128.hip",
           "decode_same_d64.hip", "decode_u3_d64.hip", "decode_fp8_d64.hip",
           "decode_e5m2_d128.hip", "decode_i8_d128.hip", "decode_e5m2_d64.hip", "decode_i8_d64.hip"]
ARCH = "gfx950"
# test-only kernels (exhaustive checks of internal arithmetic), built beside their tests
TEST_KERNELS = [os.path.join(ROOT, "tests", "gpu_kernels", "fp8_checks.hip")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedkv.so)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-I", os.path.join(ROOT, "include"),
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + common_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libpagedkv.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    for src in TEST_KERNELS:
        _build_test_kernel(src, verbose)
    return OUT


def test_kernel_path(src: str) -> str:
    return os.path.join(os.path.dirname(src), "libpkv_" + os.path.splitext(os.path.basename(src))[0] + ".so")


def _build_test_kernel(src: str, verbose: bool) -> str:
    out = test_kernel_path(src)
    cmd = [hipcc()] + common_flags() + ["-shared", "-x", "hip", src, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
