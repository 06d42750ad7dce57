"""Builds liblrmoe.so (HIP, gfx950) in-tree with hipcc.

``python -m load_recalibrated_expert_amd.build`` or ``build_library()``. Objects go to
``_build/`` under the repository root; the shared library lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblrmoe.so")
SOURCES = ["lrmoe_abi.hip", "score.hip", "select.hip", "compact.hip", "gemm.hip", "scatter.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is noise
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        return _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(jobs or min(8, len(SOURCES))) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
