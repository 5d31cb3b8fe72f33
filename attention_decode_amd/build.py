"""Build libtq.so in-tree with hipcc for gfx950 (no JIT, no torch extension).

    python -m attention_decode_amd.build

Every translation unit (C ABI, host math, HIP kernels) goes into one shared
library next to this file.  Device code is compiled with packed fp32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtq.so")
SOURCES = ["api.cpp", "host_math.cpp", "k_keys.hip", "k_values.hip", "k_decode.hip", "k_attend_mfma.hip",
           "k_dequant.hip", "k_block.hip", "scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Per-file code generation options (none at present).
FILE_FLAGS: dict[str, list[str]] = {}


def compile_cmd(src: str, obj: str) -> list[str]:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    return [hipcc(), *lang, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *FILE_FLAGS.get(os.path.basename(src), []),
            "-I", os.path.join(PKG, "..", "include"), "-c", src, "-o", obj]


CALIB = os.path.join(PKG, "calib_read")
CALIB_PROGRAMS = ("calib_read", "calib_mfma")


def calib_cmd(out: str, name: str = "calib_read") -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            os.path.join(PKG, name + ".hip"), "-o", out]


def build(verbose: bool = False, jobs: int = 8) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for name in SOURCES:
        src = os.path.join(CSRC, name)
        obj = os.path.join(objdir, name + ".o")
        objs.append(obj)
        cmd = compile_cmd(src, obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for name, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature name; harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append(name)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # calibration programs: streaming read (bench.py --calib-read) and matrix
    # cores (bench.py --calib-mfma)
    for name in CALIB_PROGRAMS:
        prog = os.path.join(PKG, name)
        r = subprocess.run(calib_cmd(prog + ".tmp", name), stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            print(r.stdout.decode(errors="replace"), file=sys.stderr)
            raise RuntimeError(f"hipcc failed for {name}.hip")
        os.replace(prog + ".tmp", prog)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
