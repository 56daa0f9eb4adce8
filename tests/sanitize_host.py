"""Run the CPU test tier with the host code under AddressSanitizer + UndefinedBehaviorSanitizer.

Builds two instrumented copies next to the normal ones (both .so files are build output):
  * oracle/liboracle_san.so -- the C oracle, clang with -fsanitize=address,undefined;
  * block_scaled_precision_mxfp8_amd/libbsq_san.so -- the library with its host code (the
    C ABI's argument validation and the launchers) instrumented; the device code is built
    exactly as in the product and is not instrumented (no GPU sanitizer is used).
then runs ``pytest -m "not gpu"`` in a child process with clang's ASan runtime preloaded
and BSQ_TEST_SANITIZED=1, which makes tests/conftest.py load the instrumented copies.
Undefined behaviour aborts (no recovery); leak checking is off (the interpreter itself is not
instrumented and keeps its allocations until exit).

    python tests/sanitize_host.py [extra pytest arguments]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

LLVM = "/opt/rocm/llvm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    found = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not found:
        raise SystemExit("clang's ASan runtime was not found under %s" % LLVM)
    return found[-1]


def build_oracle(verbose: bool = True) -> str:
    out = os.path.join(ROOT, "oracle", "liboracle_san.so")
    cmd = [os.path.join(LLVM, "bin", "clang"), "-O1", *SAN, "-shared-libsan", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-Werror", "-o", out, os.path.join(ROOT, "oracle", "bsq_oracle.c"), "-lm",
           "-L" + os.path.join(LLVM, "lib"), "-Wl,-rpath," + os.path.join(LLVM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def build_library(verbose: bool = True) -> str:
    from block_scaled_precision_mxfp8_amd import build as bsq_build

    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    objs = []
    for src in bsq_build.SOURCES:
        obj = os.path.join(bsq_build.CSRC, os.path.splitext(src)[0] + "_san.o")
        cmd = [bsq_build.hipcc(), *bsq_build.HIPCC_FLAGS, *host_san, "-x", "hip", "-c",
               os.path.join(bsq_build.CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    out = os.path.join(bsq_build.HERE, "libbsq_san.so")
    cmd = [os.path.join(LLVM, "bin", "clang++"), "-shared", *SAN, "-shared-libsan", "-o", out, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    for o in objs:
        os.remove(o)
    return out


def main(argv) -> int:
    import tempfile

    build_oracle()
    build_library()
    logs = tempfile.mkdtemp(prefix="bsq_san_")
    env = dict(os.environ)
    # the ASan runtime must come first; an LD_PRELOAD already set stays after it
    env["LD_PRELOAD"] = " ".join(x for x in (asan_runtime(), os.environ.get("LD_PRELOAD", "")) if x)
    # reports go to files: pytest captures the test's stderr, which an abort would lose
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:log_path=%s/asan" % logs
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:log_path=%s/ubsan" % logs
    env["BSQ_TEST_SANITIZED"] = "1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", *argv]
    print("LD_PRELOAD=%s %s" % (env["LD_PRELOAD"], " ".join(cmd)), flush=True)
    rc = subprocess.call(cmd, env=env, cwd=ROOT)
    reports = sorted(glob.glob(os.path.join(logs, "*")))
    for path in reports:
        print("==== %s" % path)
        print(open(path).read())
    print("sanitizer reports: %d" % len(reports), flush=True)
    return rc if rc != 0 else (1 if reports else 0)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
