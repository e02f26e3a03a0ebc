"""Build libw4a8.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m w4a8_quantized_linear_amd.build

Every .hip file under csrc/ is compiled with hipcc for gfx950 and linked into
w4a8_quantized_linear_amd/libw4a8.so.  No fast-math: the quantizers rely on
IEEE division and round-half-even.  Packed fp32 instructions are disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libw4a8.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("W4A8_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under %s" % CSRC)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built %s" % LIB)
    return LIB


if __name__ == "__main__":
    build()
