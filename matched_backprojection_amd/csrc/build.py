"""Build the HIP library ``libmbp.so`` for gfx950 with hipcc (in-tree).

All device code is compiled with packed-FP32 instructions disabled and with hardware float
atomics (``-munsafe-fp-atomics``: a float atomicAdd lowers to one global atomic add instead
of a compare-and-swap loop).
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmbp.so")
SOURCES = [os.path.join(HERE, "kernels.hip"), os.path.join(HERE, "plan.cpp"),
           os.path.join(HERE, "solver.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("MBP_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", HERE,
]


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libmbp.so`` (always recompiles)."""
    objs = []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", os.path.basename(src) + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [HIPCC, *HIP_FLAGS, "-x", "hip", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB




HOSTCHECK_SRC = os.path.join(HERE, "hostcheck.cpp")
HOSTCHECK_LIB = os.path.join(HERE, "_build", "libmbp_hostcheck.so")


def build_hostcheck(verbose: bool = False) -> str:
    """Compile the CPU replay of the walks (test harness) with g++."""
    os.makedirs(os.path.dirname(HOSTCHECK_LIB), exist_ok=True)
    tmp = HOSTCHECK_LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas",
           "-I", HERE, "-o", tmp, HOSTCHECK_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, HOSTCHECK_LIB)
    return HOSTCHECK_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_hostcheck(verbose="-v" in sys.argv))
