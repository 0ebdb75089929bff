"""Build libfp8moe.so in-tree for gfx950 with hipcc.

Each HIP source compiles to an object (in parallel), the host-only
validation unit compiles with the host C++ compiler, and everything links into
``mxfp8_quantized_moe_amd/libfp8moe.so``.  Always rebuilds.

Flags: no fast-math and no flush-to-zero (the quantizers need IEEE division,
multiplication and subnormals); packed fp32 instructions are disabled for the
device code.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8moe.so")

HIP_SOURCES = ["api.hip", "quant_rowwise.hip", "quant_colwise.hip", "quant_mx.hip", "gemm_grouped.hip", "gemm_bf16.hip",
               "swiglu_quant.hip", "moe_route.hip",
               "quant_tensorwise.hip", "blockwise.hip"]
HOST_SOURCES = ["validate.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc", "-I", os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stdout + r.stderr


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s.replace(".cpp", ".o"))
        cmds.append([shutil.which("g++") or "g++", *HOST_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    with cf.ThreadPoolExecutor(jobs) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
