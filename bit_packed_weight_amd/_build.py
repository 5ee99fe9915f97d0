"""Build libbpw.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m bit_packed_weight_amd._build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the shared library is written
next to this file so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbpw.so")

SOURCES = ["api.cpp", "prepare.cpp", "quant.hip", "gemv.hip", "gemm_i8.hip", "gemm_w4.hip", "probe.hip",
           "scratch.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
          "-Wno-pass-failed", "-I", os.path.join(ROOT, "include")]
# Packed fp32 instructions stay off: the compiler must not form v_pk_*_f32.
# Kernel arguments are preloaded into SGPRs (up to 16 dwords), so a kernel
# starts without waiting on argument loads; that wait is a visible part of a
# few-microsecond GEMV. The code object keeps the ordinary loads for firmware
# without preloading.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=16"]
# The int8 GEMM folds every MFMA result with VALU instructions, which cannot
# read AGPRs: its MFMA results must be allocated in VGPRs.
EXTRA = {"gemm_i8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libbpw.so")
    return path


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += DEVICE + EXTRA.get(src, [])
    cmd += ["-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", *DEVICE, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
