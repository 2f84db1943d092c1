"""The public header is a C interface: a C11 client (tests/native/abi_c_client.c)
compiles against include/w4a4.h with warnings as errors, links the built
libw4a4.so and calls entry points that need no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rotation_w4a4_quantization_amd")
SRC = os.path.join(ROOT, "tests", "native", "abi_c_client.c")


def test_c_client_builds_links_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(PKG, "libw4a4.so")):
        pytest.skip("libw4a4.so is not built")
    exe = str(tmp_path / "abi_c_client")
    build = subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                            SRC, "-L", PKG, "-lw4a4", f"-Wl,-rpath,{PKG}", "-o", exe],
                           capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and "c client ok" in run.stdout, run.stdout + run.stderr
