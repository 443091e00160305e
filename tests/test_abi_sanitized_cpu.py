"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU): kvq_api.hip is built with
both sanitizers into a small driver (tests/sanitize/abi_validation.cpp) that
runs the error cases of test_abi_cpu.py plus size extremes against launcher
stand-ins that abort if a check lets a call through. Any sanitizer report or
status mismatch fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def test_validation_paths_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_validation")
    # each sanitizer flag applies to the host pass only (-Xarch_host right before it)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Wno-unused-command-line-argument", "-Wno-inline-asm",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "quantized_decode_attention_03_amd", "csrc"), "-o", exe,
           os.path.join(ROOT, "tests", "sanitize", "abi_validation.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           os.path.join(ROOT, "quantized_decode_attention_03_amd", "csrc", "kvq_api.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "all validation checks passed" in r.stdout
