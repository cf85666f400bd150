"""Run the CPU test suite against host-sanitized builds (AddressSanitizer + UBSan).

Builds the host code of libmbp.so (validation, plans, scheduling), the CPU replay of the
walks and the fp64 oracle with clang's AddressSanitizer and UndefinedBehaviorSanitizer into
their ``_build/san/`` folders, then runs ``pytest -m "not gpu"`` in a child process that
preloads clang's sanitizer runtime and selects those builds (MBP_SANITIZED=1). Any
sanitizer report aborts the run with a non-zero status.

    python tests/run_sanitized.py [extra pytest arguments]
"""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def main() -> int:
    spec = importlib.util.spec_from_file_location(
        "mbp_build", os.path.join(ROOT, "matched_backprojection_amd", "csrc", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    print(b.build(sanitize=True), flush=True)
    print(b.build_hostcheck(sanitize=True), flush=True)
    sys.path.insert(0, ROOT)
    from oracle import oracle as O
    print(O.build(sanitize=True), flush=True)
    env = dict(os.environ)
    env["MBP_SANITIZED"] = "1"
    env["LD_PRELOAD"] = RUNTIME
    # python itself is not instrumented: its allocations are not leaks of the code under test
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           *sys.argv[1:]]
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
