"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, run on
the CPU:

* the host side of libkvc's C ABI (kvc_api.hip: argument validation,
  workspace layout, dispatch) linked against stub launchers
  (tests/sanitize/launch_stubs.cpp) and driven by tests/sanitize/abi_host_check.c
  with fake device pointers -- every entry point's validation paths, the host
  helpers, 64-bit workspace sizes;
* the CPU oracle (oracle/oracle.c) under its pins (tests/test_oracle_pins.py),
  loaded through ORACLE_LIB with the sanitizer runtimes preloaded.

Any sanitizer report aborts the program (-fno-sanitize-recover=all), so a
clean exit is the check.  Device code is built as usual; only host code is
instrumented."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)
                                     and shutil.which("gcc")),
                                reason="hipcc, clang and gcc are needed")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_abi_host_side_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "compressed_decode_attention_amd", "csrc")]
    hip = [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", *SAN, *inc]
    api = str(tmp_path / "api.o")
    stubs = str(tmp_path / "stubs.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "abi_check")
    _run([*hip, "-c", os.path.join(ROOT, "compressed_decode_attention_amd", "csrc",
                                   "kvc_api.hip"), "-o", api])
    _run([*hip, "-x", "hip", "-c", os.path.join(HERE, "launch_stubs.cpp"), "-o", stubs])
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "abi_host_check.c"),
          "-o", drv])
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", api, stubs, drv, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([exe], env=env, timeout=120)
    assert "0 failure(s)" in r.stdout


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"])
    rt = ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True,
                                 text=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
              os.path.join(ROOT, "tests", "test_oracle_pins.py")], env=env, cwd=ROOT, timeout=600)
    assert " passed" in r.stdout
