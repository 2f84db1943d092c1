"""The host validation unit (csrc/validate.h, plain C++ shared by every
entry point) built on its own with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU: every argument rule, the
architecture rule's wrong-device branch, and sizes that would overflow a
naive product."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rotation_w4a4_quantization_amd", "csrc")
SELFTEST = os.path.join(ROOT, "tests", "native", "validate_selftest.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validate_unit_under_sanitizers(tmp_path):
    exe = str(tmp_path / "validate_selftest")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", CSRC, SELFTEST, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "validate selftest ok" in run.stdout
