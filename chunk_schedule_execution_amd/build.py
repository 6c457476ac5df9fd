"""Build libccl.so in-tree with hipcc for gfx950.

One shared library holds the host compiler, the plan runtime, the C entry points and
the executor kernel. Host sources are plain C++17; the kernel source is HIP. Every
file is compiled with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libccl.so")
BUILD = os.path.join(ROOT, "_build")

HOST_SOURCES = ["compiler.cpp", "simulate.cpp", "capi.cpp", "tune.cpp"]
DEVICE_SOURCES = ["executor.hip"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include"]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-gpu-rdc", "-mcode-object-version=5"]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stdout + r.stderr


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    for s in HOST_SOURCES:
        jobs.append([cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, s),
                     "-o", os.path.join(BUILD, s + ".o")])
    for s in DEVICE_SOURCES:
        jobs.append([cc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + DEVICE_SOURCES]
    tmp = LIB + ".tmp"
    outs.append(_run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
