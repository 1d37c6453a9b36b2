"""Builds libdeltacome.so in-tree (gfx950 device code + host C++).

    python -m tenant_rank_serving_amd.build

HIP sources go through hipcc for --offload-arch=gfx950 with packed-fp32
instructions disabled; host-only C++ goes through g++.  Objects land in
_build/ at the repository root; the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdeltacome.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", "-Wno-unused-variable",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n%s\n%s" % (" ".join(cmd), p.stdout))
    return p.stdout


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libdeltacome.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = _sources()
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        cmds.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
