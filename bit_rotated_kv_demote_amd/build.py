"""Build libamdoscar.so in-tree with hipcc for gfx950 (every call rebuilds)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libamdoscar.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
                # never emit packed-fp32 VALU instructions
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # LDS use stays exactly what the kernels declare
                "-mllvm", "-disable-promote-alloca-to-lds",
                # matrix-core accumulators in VGPRs: no AGPR <-> VGPR copies in
                # loops whose accumulators are also touched by vector code
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
HIP_SOURCES = ["demote.hip", "decode.hip", "decode_bf16.hip", "merge.hip", "noalloc.hip"]
HOST_HIP_SOURCES = ["oscar_api.cpp"]      # host code that needs the HIP runtime headers
HOST_SOURCES = ["calibrate.cpp"]          # plain C++


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return cmd[-1]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        jobs.append([HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, s), "-o",
                     os.path.join(BUILD, s + ".o")])
    for s in HOST_HIP_SOURCES:
        jobs.append([HIPCC, "-O2", "-std=c++17", "-fPIC", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                     "-I/opt/rocm/include", "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    for s in HOST_SOURCES:
        jobs.append(["g++", "-O3", "-std=c++17", "-fPIC", "-pthread", "-c", os.path.join(CSRC, s), "-o",
                     os.path.join(BUILD, s + ".o")])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
