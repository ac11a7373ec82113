"""Build libozk.so in-tree with hipcc for gfx950.

Usage: python -m fp64_gemm_emulation_ozk_amd.build  (or call build_library()).
Every source is compiled on each call (one hipcc process per file, in parallel), then
linked into fp64_gemm_emulation_ozk_amd/libozk.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libozk.so")

ARCH = "gfx950"
DEVICE_SOURCES = ["deconstruct.hip", "gemm_i8.hip", "crt.hip", "gemv.hip", "gemv_digits.hip",
                  "fp4limb.hip", "fp4awe.hip", "fp4awe4.hip", "spmv.hip", "noalloc.hip"]
HOST_SOURCES = ["rns_host.cpp", "api.cpp"]

COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                "-ffp-contract=off", "-I", os.path.join(ROOT, "include")]
# Packed fp32 instructions are disabled for all device code.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"]
# Per-source additions.  The CRT reads every MFMA result straight into VALU work
# (cross-lane swaps, conversions): results in VGPRs save a copy out of the AGPRs each.
EXTRA_FLAGS = {"crt.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               # the 6-product encoding table is searched at compile time
               "fp4awe.hip": ["-fconstexpr-steps=16777216"],
               "fp4awe4.hip": ["-fconstexpr-steps=16777216"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS]
    cmd += DEVICE_FLAGS
    cmd += EXTRA_FLAGS.get(src, [])
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = [s for s in DEVICE_SOURCES + HOST_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(sources)} sources", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build_library()
