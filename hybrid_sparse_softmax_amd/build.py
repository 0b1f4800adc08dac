"""Builds libstill.so (HIP kernels + C-ABI layer) for gfx950 with hipcc.

Run ``python -m hybrid_sparse_softmax_amd.build``; objects go to ``_build/``
at the repository root and the library to ``hybrid_sparse_softmax_amd/_lib``.
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
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libstill.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["still_api.cpp", "general.hip", "decode.hip", "decode_fast.hip", "prefill_mfma.hip",
           "backward.hip", "backward_mfma.hip", "utility.hip"]
# sources whose matrix-core accumulators stay live across a whole loop and are
# best left to the compiler's register-file choice (accumulation registers)
FREE_ACC = {"backward_mfma.hip"}

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    # keep MFMA accumulators in ordinary VGPRs: with the default heuristic the
    # forward's main loop copied its whole accumulator tile between register
    # files on every iteration
    extra = [] if src in FREE_ACC else ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
