"""Build libdfc.so in place (host codec with g++, gfx950 decoder with hipcc),
and libdfc_probe.so, the benchmark's streaming-ceiling kernel.

Usage: python -m lossless_entropy_coded_dfc_amd.csrc.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libdfc.so")
# the benchmark's streaming ceiling (not part of the codec)
PROBE_OUT = os.path.join(PKG, "libdfc_probe.so")
ARCH = "gfx950"

# Packed FP32 instructions are kept out of every HIP object.  Unaligned
# access mode is switched off so the compiler never merges narrow LDS stores
# into wide ones at unaligned addresses: gfx950 executes those one lane at a
# time.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xclang", "-target-feature", "-Xclang", "-unaligned-access-mode",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdfc)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, out: str = OUT) -> str:
    """Compile every source and link libdfc.so next to the package."""
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", HERE]
    host_objs = []
    for name in ("dfc_host", "dfc_ans_host"):
        obj = os.path.join(objdir, name + ".o")
        _run(["g++", *CXX_FLAGS, *inc, "-c", os.path.join(HERE, name + ".cpp"), "-o", obj], verbose)
        host_objs.append(obj)
    dev_objs = []
    for name in ("dfc_decode", "dfc_ans", "dfc_gemm", "dfc_encode_gpu"):
        obj = os.path.join(objdir, name + ".o")
        _run([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(HERE, name + ".hip"), "-o", obj], verbose)
        dev_objs.append(obj)
    tmp = out + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *host_objs, *dev_objs, "-pthread"], verbose)
    os.replace(tmp, out)
    if out == OUT:
        tmp = PROBE_OUT + ".tmp"
        _run([hipcc, *HIP_FLAGS, "-shared", "-o", tmp, os.path.join(HERE, "dfc_probe.hip")], verbose)
        os.replace(tmp, PROBE_OUT)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
