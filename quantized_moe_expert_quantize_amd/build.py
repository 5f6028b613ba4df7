"""Build libftq.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_moe_expert_quantize_amd.build

Every call compiles every source again (no timestamp-based reuse: a stale
object silently reused after a header swap is exactly the trap FreeToken PR
#185 warns about in its Test section).  The source hash is written next to the
library so that a run can report which sources it executed.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libftq.so")
HASH_FILE = os.path.join(PKG, "libftq.sha256")
BUILD_DIR = os.path.join(ROOT, "_build", "ftq")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are kept out of generated code on purpose.  No implicit
# contraction: every fused multiply-add in the kernels is written out (fmaf),
# and a product that feeds an fp16 conversion must round to fp32 first.  No
# type-based alias analysis: the kernels write LDS and global staging buffers
# as 16-byte vectors and read them back as words (and the other way round), and
# with strict aliasing the compiler may move such a read above the write.
FLAGS = ["-std=c++17", "-O3", "-fPIC", "-ffp-contract=off", "-fno-strict-aliasing", "-Wall", "-Wno-unused-function",
         "-Wno-cuda-compat", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]


# Per-file flags.  grouped.hip: machine-level sinking would move the
# scale-accumulates of the warp-specialised kernel out of the slots between its
# matrix products (into the block after a stage's counter update), which
# serialises them and multiplies the live registers.
FILE_FLAGS = {"grouped.hip": ["-mllvm", "-disable-machine-sink"]}


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp")):
            out.append(os.path.join(CSRC, name))
    return out


def source_hash() -> str:
    h = hashlib.sha256()
    files = sources() + [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]
    files.append(os.path.join(INCLUDE, "ftq.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the gfx950 target feature: drop that noise
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and noise not in l]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(HASH_FILE, "w") as fh:
        fh.write(source_hash() + "\n")
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
