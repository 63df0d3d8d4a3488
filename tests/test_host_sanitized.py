"""Sanitizer builds of the host code (CPU only, no GPU): the C oracle and
the C-ABI state machine (kivi_api.cpp) with its kernel launchers and HIP
queries replaced by host stubs (tests/host/stub_launch.cpp), both built with
AddressSanitizer and UndefinedBehaviorSanitizer by g++/gcc and run to
completion.  The state-machine program checks the error contract: launch
failures injected by the stubs return KIVI_ERR_HIP and poison the handle, a
failed device query leaves the cache unchanged, and the fused decode step
plans the state after its append before its first launch."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
BUILD = os.path.join(HOST, "_build")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _build(cmd):
    os.makedirs(BUILD, exist_ok=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_state_machine_contract_sanitized():
    exe = os.path.join(BUILD, "contract_test")
    _build(["g++", "-std=c++17"] + SAN + [
        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
        os.path.join(ROOT, "kv_cache_bit_kivi_amd", "csrc", "kivi_api.cpp"),
        os.path.join(HOST, "stub_launch.cpp"), os.path.join(HOST, "contract_test.cpp"), "-o", exe])
    out = _run(exe)
    assert "checks passed" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_sanitized():
    exe = os.path.join(BUILD, "oracle_driver")
    _build(["gcc", "-std=c11"] + SAN + [
        "-ffp-contract=off", "-fopenmp", os.path.join(ROOT, "oracle", "kivi_oracle.c"),
        os.path.join(HOST, "oracle_driver.c"), "-o", exe, "-lm"])
    assert "ok" in _run(exe)
