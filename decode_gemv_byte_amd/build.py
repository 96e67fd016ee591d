"""Build libnwc.so (host codec + gfx950 HIP kernels) in-tree with hipcc.

    python decode_gemv_byte_amd/build.py

(run as a script: importing the package would load the library first).

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnwc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# kernarg preload: a kernel's first 7 arguments arrive in scalar registers at
# launch (k_gemv's job boundaries), a memory round trip less before its first
# tile load; the compiler keeps a loading prologue for firmware without it
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=7"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in ("host_codec.cpp", "kernels.hip", "prefill.cpp"):
        obj = os.path.join(BUILD, src + ".o")
        host = ["-x", "c++", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]  # host code (HIP runtime API only)
        cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else host) + \
              ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs + \
          ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lhipblaslt", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
