"""The library's host code -- the C ABI's argument checks, workspace sizing and dispatch -- under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The library is rebuilt with only its host code instrumented (device code as usual) and the host-only ABI
tests and the binding's checks run against it in a child process with the sanitizer runtime preloaded.
Every case there fails validation before any launch, so no GPU is needed; a sanitizer report (out-of-bounds
access, overflow, misaligned load, ...) fails the test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_host_checks_under_asan_and_ubsan():
    from mla_latent_kv_cache_amd import build

    lib = build.build_host_sanitized(verbose=False)
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(), MLA_LATENT_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=97",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_abi_host.py", "tests/test_binding_validation.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out and "failed" not in out, out[-3000:]
