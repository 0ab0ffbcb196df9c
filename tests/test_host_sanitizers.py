"""Host code and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- libfdec's host code (api.cpp, plan.cpp) is built with g++ and both sanitizers
  against host-only stand-ins for the HIP runtime and the kernel launchers
  (tests/host/stubs.cpp), and driven through every entry point over seeded random
  shapes (tests/host/drive_host.py): the stand-ins abort when a launch would touch
  a range outside the buffers the caller passed, or write overlapping workspace
  ranges, or write the fused path's arrival counters from any other launch.
- The fp64 oracle (oracle/oracle.c) is built into a driver (tests/host/drive_oracle.c)
  with both sanitizers and exact-size buffers, over seeded random cases, checking
  its own identities on the way (merged partials = decode, one-token multi = decode).
Any sanitizer report aborts the child process and fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "decode_attention_fdec_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime():
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


needs_gcc = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None or _asan_runtime() is None,
                               reason="g++ / gcc with the AddressSanitizer runtime not available")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{out[-4000:]}"
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


@needs_gcc
def test_host_code_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libfdec_host.so")
    _run(["g++", "-std=c++17", *SAN, "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{os.path.join(ROOT, 'include')}", os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
          os.path.join(HOST, "stubs.cpp"), "-o", lib])
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run([sys.executable, os.path.join(HOST, "drive_host.py"), lib, "800"], env=env)
    assert "host sweep ok" in out


@needs_gcc
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "drive_oracle")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(HOST, "drive_oracle.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    out = _run([exe, "200"], env=env)
    assert "oracle sweep ok" in out
