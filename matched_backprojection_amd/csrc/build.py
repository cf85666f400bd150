"""Build the HIP library ``libmbp.so`` for gfx950 with hipcc (in-tree).

All device code is compiled with packed-FP32 instructions disabled and with hardware float
atomics (``-munsafe-fp-atomics``: a float atomicAdd lowers to one global atomic add instead
of a compare-and-swap loop).

``sanitize=True`` builds host-sanitized copies into ``_build/san/`` instead: the host code of
``libmbp.so`` (validation, plans, scheduling) and the CPU replay of the walks with
AddressSanitizer and UndefinedBehaviorSanitizer (clang's runtime, preloaded by the process
that loads them; device code is built as usual). ``tests/run_sanitized.py`` drives it.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmbp.so")
SAN_DIR = os.path.join(HERE, "_build", "san")
SOURCES = [os.path.join(HERE, "kernels.hip"), os.path.join(HERE, "plan.cpp"),
           os.path.join(HERE, "solver.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ARCH = os.environ.get("MBP_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", HERE,
]
# host-only sanitizers: each flag applies to the host compilation alone
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link ``libmbp.so`` (always recompiles)."""
    out_dir = SAN_DIR if sanitize else os.path.join(HERE, "_build")
    lib = os.path.join(SAN_DIR, "libmbp.so") if sanitize else LIB
    extra = HOST_SAN_FLAGS if sanitize else []
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        os.makedirs(out_dir, exist_ok=True)
        cmd = [HIPCC, *HIP_FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


HOSTCHECK_SRC = os.path.join(HERE, "hostcheck.cpp")
HOSTCHECK_LIB = os.path.join(HERE, "_build", "libmbp_hostcheck.so")


def build_hostcheck(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile the CPU replay of the walks (test harness): g++, or clang++ with ASan and UBSan."""
    lib = os.path.join(SAN_DIR, "libmbp_hostcheck.so") if sanitize else HOSTCHECK_LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp%d" % os.getpid()
    if sanitize:
        cmd = [CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-Wall",
               "-Wno-unknown-pragmas", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
               "-fno-sanitize-recover=all", "-I", HERE, "-o", tmp, HOSTCHECK_SRC]
    else:
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-Wall",
               "-Wno-unknown-pragmas", "-I", HERE, "-o", tmp, HOSTCHECK_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    san = "--sanitize" in sys.argv
    print(build(verbose="-v" in sys.argv, sanitize=san))
    print(build_hostcheck(verbose="-v" in sys.argv, sanitize=san))
