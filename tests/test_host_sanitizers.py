"""The host ABI tests (tests/test_abi_host.py) again, on a build of the library whose host
code (argument checks, workspace layouts, launch set-up of the C ABI) carries
AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code is the same.  Any report
of either sanitizer fails the test.  CPU only: the checks run before any GPU work."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_library():
    from long_context_decode_kvfetch_amd import build
    path = build.SANITIZED_LIB
    stale = True
    if os.path.exists(path):
        # the hash compiled into a build: the first 64 hex digits after its marker string
        with open(path, "rb") as f:
            stale = build.source_hash().encode() not in f.read()
    if stale:
        build.build(sanitize_host=True)
    return path, build.sanitizer_runtime()


def test_sanitized_build_is_instrumented():
    path, _ = _sanitized_library()
    out = subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in out and "__ubsan_handle" in out


def test_host_abi_under_address_and_undefined_sanitizers():
    path, runtime = _sanitized_library()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, VERKV_LIBRARY=path,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"),
                          "-q", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = res.stdout + res.stderr
    assert "AddressSanitizer" not in log, log[-4000:]
    assert "runtime error:" not in log, log[-4000:]
    assert res.returncode == 0, log[-4000:]
    assert " passed" in log
