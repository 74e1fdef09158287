"""Build the gfx950 shared library ``libssm_mi355x.so`` in-tree with hipcc.

Every ``csrc/*.hip`` file and ``csrc/abi.cpp`` is compiled to an object with
``hipcc --offload-arch=gfx950`` (packed-fp32 instructions disabled), then linked
with ``-shared``.  Objects go to ``_build/`` next to this file; the library is
written beside the package modules so it is picked up from the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_mi355x.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "abi.cpp")]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    p = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
