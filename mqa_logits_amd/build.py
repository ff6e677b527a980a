"""Build libmqa_logits.so in-tree with hipcc for gfx950.

Usage: python mqa_logits_amd/build.py   (or __graft_entry__.build())

Run it by path: importing the package loads the library this script makes.

Every call recompiles.  Objects go to mqa_logits_amd/_build/, the shared
library to mqa_logits_amd/libmqa_logits.so.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmqa_logits.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dense.hip", "dense_bf16.hip", "dense_sched.hip", "dense_sched_bf16.hip",
           "topk.hip", "paged.hip", "api.cpp"]
# measurement aid for bench.py, linked into a library of its own
PROBE_SOURCES = ["peak.hip"]
PROBE_LIB = os.path.join(PKG, "libmqa_peak.so")

# Packed fp32 VALU forms are kept out of the generated code on purpose.
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # Accumulators in VGPRs (the Q operands are pinned to AGPRs), and no NaN
    # canonicalisation in front of each ReLU max.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    pobjs = [_compile(src) for src in PROBE_SOURCES]
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *pobjs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
