#!/usr/bin/env python3
"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU-side code.

Not a pytest module (run it by hand; it needs no GPU):

    python tests/host_sanitizers.py [--keep]

1. oracle/oracle.c is built with gcc -fsanitize=address,undefined into a
   scratch directory, and the CPU suite (pytest -m "not gpu") runs against it
   with gcc's ASan runtime preloaded (ORACLE_LIB_PATH selects the build).
2. libftq's host code (argument validation, path choice, workspace and launch
   planning) is built with the sanitizers on the host pass only (each
   -fsanitize= follows -Xarch_host; the gfx950 device code is unchanged), and
   the CPU suite runs again with clang's ASan runtime preloaded (FTQ_LIB_PATH
   selects the build).  Without a GPU those tests reach every host entry
   point that does not launch: size and pointer checks, workspace sizes, the
   path rule and the GEMV plan, and the errors they return.

Leak detection is off (the Python interpreter itself is not leak-clean); any
other ASan report or UBSan diagnostic fails the run.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from quantized_moe_expert_quantize_amd import build as ftq_build  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, env=env)


def clang_asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's ASan runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def build_oracle(out: str) -> str:
    lib = os.path.join(out, "liboracle_san.so")
    run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
         "-shared", "-fPIC", os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"])
    return lib


def build_libftq(out: str) -> str:
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        cmd = [ftq_build.HIPCC, *ftq_build.FLAGS, *ftq_build.FILE_FLAGS.get(os.path.basename(src), []), *host_san,
               "-x", "hip", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    srcs = ftq_build.sources()
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(out, "libftq_san.so")
    run([ftq_build.HIPCC, f"--offload-arch={ftq_build.ARCH}", "-shared", "-fPIC", *host_san, "-shared-libsan",
         *objs, "-o", lib])
    return lib


PLANTED = r"""
#include <stdlib.h>
int planted_overflow(int n) { int* v = (int*)malloc(sizeof(int) * n); int s = v[n]; free(v); return s; }
"""


def self_check(out: str, compiler: list, env: dict, name: str) -> None:
    """The harness must catch a planted heap overflow in a library it loads the
    same way (a CPU-only check that the preloaded runtime is active)."""
    src = os.path.join(out, name + ".c")
    lib = os.path.join(out, name + ".so")
    with open(src, "w") as fh:
        fh.write(PLANTED)
    run([*compiler, "-shared", "-fPIC", src, "-o", lib])
    code = f"import ctypes; ctypes.CDLL({lib!r}).planted_overflow(4)"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    if r.returncode == 0 or "heap-buffer-overflow" not in r.stderr:
        raise RuntimeError(f"{name}: the planted overflow was not reported (exit {r.returncode})")
    print(f"{name}: planted overflow reported, as it should be", flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--keep", action="store_true", help="keep the scratch directory")
    args = ap.parse_args()
    out = tempfile.mkdtemp(prefix="ftq_sanitizers_")
    pytest = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
              "-p", "no:cacheprovider"]
    try:
        oracle_lib = build_oracle(out)
        gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                                  check=True).stdout.strip()
        env = dict(os.environ, **SAN_ENV, LD_PRELOAD=gcc_asan, ORACLE_LIB_PATH=oracle_lib)
        self_check(out, ["gcc", "-g", "-fsanitize=address,undefined"], env, "planted_gcc")
        run(pytest, env)
        print("oracle under ASan + UBSan: clean", flush=True)

        ftq_lib = build_libftq(out)
        env = dict(os.environ, **SAN_ENV, LD_PRELOAD=clang_asan_runtime(), FTQ_LIB_PATH=ftq_lib)
        self_check(out, ["/opt/rocm/llvm/bin/clang", "-g", "-fsanitize=address,undefined", "-shared-libsan"], env,
                   "planted_clang")
        run(pytest, env)
        print("libftq host code under ASan + UBSan: clean", flush=True)
    finally:
        if args.keep:
            print("scratch:", out)
        else:
            shutil.rmtree(out, ignore_errors=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
