"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

- The library's host side (validation, layouts, carving, the launch set-up of
  sage_api.hip), built with both sanitizers for the host only and linked with
  the normal kernel objects, runs tests/host_check/abi_driver.cpp: every entry
  point with sizes up to the limits and with every kind of bad argument.  No
  call reaches a device.
- The oracle (oracle.c), built with both sanitizers, runs its own pins (the
  oracle test files) in a child process with the ASan runtime preloaded.

Either run must end with status 0 and without a sanitizer report.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "host_check"))

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehavior")


def _env(**extra):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


def _clean(out):
    return not any(r in out for r in REPORTS)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_library_host_code_under_sanitizers():
    import build as host_build
    exe = host_build.build_abi_check()
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert _clean(out), out[-4000:]
    assert "all calls returned as expected" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_under_sanitizers():
    import build as host_build
    lib = host_build.build_oracle_san()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.exists(asan), "gcc's ASan runtime is missing"
    import oracle
    env = _env(LD_PRELOAD=asan, **{oracle.SANITIZED_LIB_ENV: lib})
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_codec.py", "test_oracle_attn.py", "test_oracle_golden.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", *tests],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert _clean(out), out[-4000:]
