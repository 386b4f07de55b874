"""Build libkq.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m quant_verify_gemv_amd.build

hipcc cross-compiles for gfx950 without a GPU. The host-side C ABI unit
(kq_api.cpp) is plain C++ and is compiled with g++; the kernels with hipcc.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkq.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are kept out of every kernel.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    tmp = tempfile.mkdtemp(prefix="kq_build_")
    try:
        obj_api = os.path.join(tmp, "kq_api.o")
        obj_k = os.path.join(tmp, "kq_kernels.o")
        # -ffp-contract=off: the host decision's float arithmetic is exactly
        # the sequence written (no fused multiply-adds)
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
              "-c", os.path.join(CSRC, "kq_api.cpp"), "-o", obj_api], verbose)
        _run([HIPCC] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c",
              os.path.join(CSRC, "kq_kernels.hip"), "-o", obj_k], verbose)
        out_tmp = LIB + f".tmp{os.getpid()}"
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "--hip-link", obj_api, obj_k,
              "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
