"""Builds the HIP library ``libmoe_mi355x.so`` for gfx950 with hipcc (in-tree).

Every translation unit is compiled for gfx950 only, with packed-fp32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``), then linked into one
shared library that exports the C ABI of ``include/moe.h``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
SOURCES = ["router.hip", "dispatch.hip", "combine.hip", "gemm_f32.hip", "gemm_bf16.hip", "moe_api.cpp"]
# measurement tooling (the memory-counter calibration copy), a library of its own
CALIB_LIB = os.path.join(PKG, "libmoe_calib.so")
CALIB_SOURCES = ["calib_copy.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build_library(extra_flags=(), verbose: bool = True) -> str:
    """Compile every source and link the shared library (and the calibration library);
    returns the layer library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, list(extra_flags)), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build_library()
