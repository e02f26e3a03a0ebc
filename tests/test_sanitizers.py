"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle, built with gcc's ASan and UBSan (every finding fatal), is
  loaded in a child process in place of the normal build (the W4A8_ORACLE_LIB
  substitution the mutation tests use) and runs the oracle's pin tests, which
  call every oracle function.
* The library's host code -- argument checks, plan selection with and
  without a workspace, the decode candidates and the selector's scores, the
  no-allocation entry point's checks -- is built by hipcc with the sanitizers
  on the host side only (device code unchanged) and linked into
  tests/sanitize/abi_driver.cpp, which calls every entry point over the
  configuration shapes and edge shapes.  No kernel is launched: every compute
  call fails validation first.

Builds are cached under _build/sanitize/ by a hash of their sources and flags.
"""
import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "w4a8_quantized_linear_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_and_ubsan():
    asan = _gcc_runtime("libasan.so")
    if asan is None or shutil.which("gcc") is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = os.path.join(ROOT, "oracle", "w4a8_oracle.c")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_asan_%s.so" % _digest([src], flags))
    if not os.path.exists(lib):
        subprocess.run(["gcc", *flags, "-o", lib + ".tmp", src, "-lm"], check=True)
        os.replace(lib + ".tmp", lib)
    env = dict(os.environ, W4A8_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    pins = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_pins.py", "test_oracle_norm_pins.py",
                                                     "test_oracle_w4a16_pins.py", "test_oracle_kv4_pins.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *pins],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail


def test_host_abi_under_asan_and_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    headers = sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(CSRC, "*.inc")) +
                     [os.path.join(ROOT, "include", "w4a8.h")])
    driver = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    key = _digest(srcs + headers + [driver], flags)
    exe = os.path.join(OUT, "abi_driver_%s" % key)
    if not os.path.exists(exe):
        objdir = os.path.join(OUT, "obj_%s" % key)
        os.makedirs(objdir, exist_ok=True)

        def compile_one(src):
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, srcs + [driver]))
        r = subprocess.run([HIPCC, *flags, *objs, "-o", exe + ".tmp"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        os.replace(exe + ".tmp", exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "abi driver: 0 failures" in out, out[-4000:]
