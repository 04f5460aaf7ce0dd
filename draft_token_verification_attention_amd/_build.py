"""Build libspecverify.so (HIP for gfx950) in-tree with hipcc.

    python draft_token_verification_attention_amd/_build.py

(run by path: importing the package needs the library this builds)
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # no packed fp32 instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    from concurrent.futures import ThreadPoolExecutor
    jobs = []
    for src in sources():
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        jobs.append(([hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj], obj))
    if verbose:
        for cmd, _ in jobs:
            print(" ".join(cmd), flush=True)
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:  # one hipcc per source file
        for f in [ex.submit(subprocess.check_call, cmd) for cmd, _ in jobs]:
            f.result()
    objs = [obj for _, obj in jobs]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "--offload-arch=" + ARCH, "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
