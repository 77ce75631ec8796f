"""The host API under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Runs tests/test_abi.py in a child process against the host-sanitized build of the
library (``python -m contextual_activation_sparsity_amd.build --sanitize``), with the ASan
runtime preloaded and UBSan set to stop at the first finding. Those tests drive every
entry point's argument validation (null pointers, bad shapes, dtypes, alignment,
workspace sizes, the no-allocation size limit) without a GPU, so the sanitizers see the
host code's whole reject path. Skipped when the sanitized build is missing or older than
the sources.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "contextual_activation_sparsity_amd")
SAN_LIB = os.path.join(PKG, "_build", "san", "libsparse_ffn_san.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def _stale():
    if not os.path.exists(SAN_LIB):
        return "sanitized build missing (python -m contextual_activation_sparsity_amd.build --sanitize)"
    srcs = glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    if max(os.path.getmtime(s) for s in srcs) > os.path.getmtime(SAN_LIB):
        return "sanitized build older than the sources"
    if not os.path.exists(CLANG):
        return "ROCm clang not found"
    return None


@pytest.mark.skipif(_stale() is not None, reason=str(_stale()))
def test_abi_under_asan_and_ubsan():
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                        check=True).stdout.strip()
    assert os.path.isabs(rt) and os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", SFN_LIBRARY=SAN_LIB)
    # the child checks that it really runs the sanitized library with ASan live
    probe = ("import ctypes\nfrom contextual_activation_sparsity_amd import binding as B\n"
             f"assert B.LIB_PATH == {SAN_LIB!r}\n"
             "assert hasattr(ctypes.CDLL(None), '__asan_report_load8')\n")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join("tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "passed" in res.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
