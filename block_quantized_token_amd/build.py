"""Build libqgemv.so in-tree: the host front with g++, the kernels with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
    # packed fp32 instructions are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive in SGPRs at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "qgemv_host.o")
    kern_o = os.path.join(BUILD, "qgemv_kernels.o")
    _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "qgemv_host.cpp"), "-o", host_o], verbose)
    quant_o = os.path.join(BUILD, "qquant_kernels.o")
    probe_o = os.path.join(BUILD, "qprobe_kernels.o")
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    # the small kernel sources compile beside the mat-vec one (which takes minutes)
    side = [subprocess.Popen([hipcc, *HIP_FLAGS, *extra_hip_flags, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj])
            for src, obj in (("qquant_kernels.hip", quant_o), ("qprobe_kernels.hip", probe_o))]
    try:
        _run([hipcc, *HIP_FLAGS, *extra_hip_flags, "-c", "-x", "hip", os.path.join(CSRC, "qgemv_kernels.hip"),
              "-o", kern_o], verbose)
    finally:
        for proc in side:
            if proc.wait() != 0:
                raise subprocess.CalledProcessError(proc.returncode, " ".join(proc.args))
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", host_o, kern_o, quant_o, probe_o, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
