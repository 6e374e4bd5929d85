"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host code (svdq_api.hip: argument checks, workspace carving, the no-allocation
entry point's size check) is built with both sanitizers for the host pass only and linked with
tests/abi_check.cpp, which drives every validation path with fake pointers and no GPU: each
call must return its status before any HIP call, with no memory error and no undefined
behaviour (an out-of-range format value, for one, must be a valid value of the enum type).
"""
import os
import shutil
import subprocess

import pytest


def test_abi_validation_under_address_and_undefined_behaviour_sanitizers():
    if not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    from bit_w4a4_quantized_amd.build import build_host_check
    exe = build_host_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK: 0 failure(s)" in r.stdout, r.stdout
