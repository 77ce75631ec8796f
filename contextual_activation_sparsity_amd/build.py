"""Build libsparse_ffn.so in-tree for gfx950 with hipcc.

    python -m contextual_activation_sparsity_amd.build [--jobs N] [--verbose] [--sanitize]

Each source is compiled to an object in ``_build/`` (in parallel), then linked into
``contextual_activation_sparsity_amd/libsparse_ffn.so`` next to the binding that loads
it. Compiles every time it is called. hipcc cross-compiles, so no GPU is needed.

``--sanitize`` instead builds ``_build/san/libsparse_ffn_san.so`` with AddressSanitizer
and UndefinedBehaviorSanitizer on the host code only (device code is built as usual).
It is for checking the host API's validation paths on the CPU: load it through the
``SFN_LIBRARY`` variable with the ASan runtime preloaded, e.g.

    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    SFN_LIBRARY=contextual_activation_sparsity_amd/_build/san/libsparse_ffn_san.so \
    python -m pytest tests/test_abi.py -q -m "not gpu"
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_ffn.so")
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libsparse_ffn_san.so")

SOURCES = ["api.cpp", "decode.hip", "svd_predict.hip", "dense_chunk.hip", "calibrate.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # packed fp32 instructions stay off: only scalar and MFMA arithmetic is emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# sanitizers on the host side only: each -fsanitize= goes to the host compilation
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsparse_ffn.so)")


def _compile(src, verbose, sanitize=False):
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, *(SANITIZE if sanitize else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; not an error
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(jobs=None, verbose=False, sanitize=False):
    os.makedirs(SAN_BUILD if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    # the sanitized library leaves the sanitizer runtime to the loading process (preloaded)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true", help="host-side ASan/UBSan build into _build/san/")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose, args.sanitize))
    return 0


if __name__ == "__main__":
    sys.exit(main())
