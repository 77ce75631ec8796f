"""The C ABI from C: tests/c_caller.c is compiled with gcc as strict C99 against
include/sparse_ffn.h, linked to libsparse_ffn.so and run. It exercises only the size
queries, the status strings and the argument checks that reject a call before any HIP
call, so it runs on the CPU and launches no kernel."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "contextual_activation_sparsity_amd")
LIB = os.path.join(PKG, "libsparse_ffn.so")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libsparse_ffn.so not built")
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_caller_links_and_sees_the_documented_statuses(tmp_path):
    exe = str(tmp_path / "c_caller")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_caller.c"), "-L", PKG, "-lsparse_ffn", f"-Wl,-rpath,{PKG}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
