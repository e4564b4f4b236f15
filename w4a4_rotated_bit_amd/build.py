"""Build the ConvRot HIP library in-tree: ``w4a4_rotated_bit_amd/libconvrot.so``.

hipcc cross-compiles for gfx950 without a GPU present.  Every HIP source is
compiled with packed-fp32 instruction selection turned off (the compiler is
free to emit v_pk_*_f32 otherwise).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_PATH = os.path.join(HERE, "libconvrot.so")
ARCH = "gfx950"

HIP_SOURCES = ["kernels.hip", "api.hip"]
CXX_SOURCES = ["host.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", CSRC, "-I", INCLUDE]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libconvrot.so; returns its path."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        out = _run([hipcc, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        _run([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
