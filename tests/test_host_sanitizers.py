"""The library's host code and the C oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

allocator.cpp, scheduler.cpp, groups.cpp, partition.cpp and status.cpp (everything in
libpa that is not a kernel or a launch) are built with g++
-fsanitize=address,undefined into a CPU-only library, oracle.c likewise with
gcc; then the CPU suites that drive them -- random operation streams against
the allocator and scheduler models, the group derivation, the oracle's pins
-- run in a child Python process with the sanitizer runtime preloaded
(PA_HOST_LIB and PA_ORACLE_LIB point the bindings at the sanitized
builds).  Any sanitizer report fails the test.  Leak checking is off: the
interpreter itself keeps allocations alive at exit."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_417_amd", "csrc")
HOST_SOURCES = ("allocator.cpp", "scheduler.cpp", "groups.cpp", "partition.cpp",
                "status.cpp")
SUITES = ("tests/test_allocator.py", "tests/test_scheduler.py", "tests/test_decode_groups.py",
          "tests/test_oracle_pins.py")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1", "-fPIC", "-shared"]


def _runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime() is None, reason="no AddressSanitizer runtime for gcc here")
def test_host_code_and_oracle_are_clean_under_asan_ubsan(tmp_path):
    host = str(tmp_path / "libpa_host_san.so")
    orc = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["g++", "-std=c++17"] + SAN + [
        "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-o", host] +
        [os.path.join(CSRC, f) for f in HOST_SOURCES])
    subprocess.check_call(["gcc", "-std=c11", "-fno-fast-math", "-ffp-contract=off"] + SAN + [
        "-o", orc, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ)
    env.update({"LD_PRELOAD": _runtime(), "PA_HOST_LIB": host, "PA_ORACLE_LIB": orc,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + list(SUITES),
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    tail = "\n".join(out.splitlines()[-30:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, tail
    assert r.returncode == 0, tail
    assert " passed" in out, tail
