"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU code (host
only; no device code is instrumented).

    python tests/sanitizers.py

1. The oracle (oracle/tq_oracle.c) built with gcc -fsanitize=address,undefined
   runs the oracle's pin tests (tests/test_oracle_*.py) with gcc's ASan
   runtime preloaded.
2. libtq's host code (csrc/api.cpp: validation, handles, workspace planning,
   the C ABI; csrc/host_math.cpp: RNG, codebook, rotations) built with clang's
   ASan and UBSan on the host side only (-Xarch_host), linked with the normal
   device objects, runs the C-ABI host tests (tests/test_abi_host.py) with
   clang's ASan runtime preloaded.

Any sanitizer report fails the run (UBSan halts on the first error).  Leak
detection is off: the Python interpreter itself does not free everything at
exit.  Build products go to a temporary directory.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_decode_amd")


def run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd, env=env, cwd=ROOT)


def main() -> int:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    out = tempfile.mkdtemp(prefix="tq_sanitize_")
    base_env = dict(os.environ)
    base_env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    base_env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"

    # 1. oracle: gcc, ASan + UBSan
    oracle_so = os.path.join(out, "liboracle_san.so")
    run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-o", oracle_so, os.path.join(ROOT, "oracle", "tq_oracle.c"), "-lm"])
    gcc_asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env = dict(base_env, LD_PRELOAD=gcc_asan, TQ_ORACLE_LIB=oracle_so)
    run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
         *sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))], env=env)

    # 2. libtq host code: clang (hipcc), host-side ASan + UBSan, with the
    # device objects of the normal build
    objdir = os.path.join(PKG, "_build")
    dev_objs = sorted(glob.glob(os.path.join(objdir, "*.hip.o")))
    if not dev_objs:
        sys.exit("build libtq first (python -m attention_decode_amd.build)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    host_objs = []
    for src in ("api.cpp", "host_math.cpp"):
        obj = os.path.join(out, src + ".o")
        run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-c", os.path.join(PKG, "csrc", src), "-o", obj])
        host_objs.append(obj)
    lib_so = os.path.join(out, "libtq_san.so")
    run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", lib_so, *host_objs, *dev_objs])
    clang_rt = glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                      "libclang_rt.asan-x86_64.so"))
    if not clang_rt:
        sys.exit("clang's ASan runtime was not found under " + rocm)
    env = dict(base_env, LD_PRELOAD=clang_rt[0], LIBTQ_PATH=lib_so)
    run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi_host.py")], env=env)
    print(f"sanitizer runs clean (build products in {out})", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
