"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* libkda's host layer (argument validation, plan and workspace arithmetic,
  error reporting): the library's sources are compiled with the sanitizers on
  their host side only (device code is built as usual and never runs here),
  and tests/sanitize/abi_driver.c calls every entry point with arguments it
  must reject before any HIP call, plus the size queries at their limits.
* the fp64 oracle: oracle/kda_oracle.c compiled with both sanitizers, and the
  oracle's pins (tests/test_oracle_pins.py) run against that build in a
  child Python process with the sanitizer runtime preloaded.

Any sanitizer report makes the child exit non-zero (recovery is off)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_05_amd", "csrc")
ROCM_LLVM = "/opt/rocm/llvm/bin"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return res.returncode, res.stdout + res.stderr


def test_host_layer_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc")
    clang = os.path.join(ROCM_LLVM, "clang++")
    if not hipcc or not os.path.exists(clang):
        pytest.skip("hipcc / ROCm clang not available")
    from linear_attention_recurrence_05_amd import build as kbuild
    # sanitizers on the host side only: each one after -Xarch_host
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    flags = [f for f in kbuild.hipcc_flags() if f != "-O3"] + ["-O1", "-g"] + host_san

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        rc, out = _run([hipcc] + flags + ["-c", "-o", obj, os.path.join(CSRC, src)])
        assert rc == 0, out
        return obj

    with ThreadPoolExecutor(len(kbuild.SOURCES)) as ex:
        objs = list(ex.map(compile_one, kbuild.SOURCES))
    lib = str(tmp_path / "libkda_san.so")
    rc, out = _run([clang, "-shared", "-o", lib] + objs + SAN[:2]
                   + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, out
    drv = str(tmp_path / "abi_driver")
    rc, out = _run([os.path.join(ROCM_LLVM, "clang"), "-g", "-O1"] + SAN
                   + ["-I", os.path.join(ROOT, "include"),
                      os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), lib,
                      f"-Wl,-rpath,{tmp_path}", "-o", drv])
    assert rc == 0, out
    rc, out = _run([drv], env={**os.environ, **SAN_ENV})
    assert rc == 0 and "OK (0 failures)" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


def test_oracle_pins_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    lib = str(tmp_path / "liboracle_san.so")
    rc, out = _run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-fno-omit-frame-pointer"] + SAN
                   + ["-o", lib, os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm"])
    assert rc == 0, out
    rc, asan = _run([gcc, "-print-file-name=libasan.so"])
    asan = asan.strip()
    if rc != 0 or not os.path.isabs(asan):
        pytest.skip("gcc's AddressSanitizer runtime not found")
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": asan, "KDA_ORACLE_LIB": lib,
           "OMP_NUM_THREADS": "4"}
    rc, out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_oracle_pins.py")], env=env, cwd=ROOT)
    assert rc == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
