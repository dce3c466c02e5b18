"""Compiles the HIP sources of the ISA library for gfx950 into an in-tree
shared library (libisa_mi355x.so next to this file).

Every HIP translation unit is built with packed-fp32 code generation
switched off, and the library exports only the extern "C" entry points
declared in include/isa.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libisa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# measurement-only probe (achievable matrix-core rate), a library of its own
PROBE_SOURCES = ["isa_probe.hip"]
PROBE_PATH = os.path.join(PKG, "libisa_probe.so")
SOURCES = ["isa_api.cpp", "isa_pool.hip", "isa_select.hip", "isa_attn.hip", "isa_attn_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}", "-Wno-unused-result"]


# The attention kernels take max/min of finite or -inf logits only; without
# NaN semantics the compiler emits v_max3 without quieting operands.
EXTRA_FLAGS = {"isa_attn.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
               "isa_attn_bwd.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + compile_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    pobjs = [_compile(src) for src in PROBE_SOURCES]
    tmp = PROBE_PATH + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + pobjs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
        print(f"built {PROBE_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
