"""Builds libtrimul.so (gfx950) in-tree from csrc/ with hipcc.

Every source is compiled on each call (no staleness guessing); objects go to
``_build/`` at the repository root and the shared library next to this file.
Run:  python -m pair_representation_amd.build
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtrimul.so")
# measurement probes (matrix-core loop, streaming kernels): a library of their
# own, loaded only by the benchmark's peaks mode
PEAKS_LIB = os.path.join(PKG, "libtrimul_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]

SOURCES = ["k1_project.hip", "k2_contract.hip", "k3_epilogue.hip", "k3b_epilogue_grad.hip", "kb_relayout.hip",
           "ka_window_attention.hip", "trimul_api.cpp"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")
    return exe


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PEAKS_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAKS_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print("built", LIB, "and", PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
