"""Compile the gfx950 HIP sources into the in-tree shared library libattn.so.

Run as ``python -m online_softmax_attn_amd.build`` (or through __graft_entry__.build()).
Each source is compiled to an object in parallel, then linked; nothing is cached between
calls, so a build always reflects the current sources.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions are kept out of all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: drop that noise
    err = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        return _run([HIPCC, *FLAGS, "-c", src, "-o", obj])

    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        for src, warn in zip(srcs, ex.map(compile_one, zip(srcs, objs))):
            if verbose and warn.strip():
                print(f"[build] {os.path.basename(src)}:\n{warn}", file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] wrote {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
