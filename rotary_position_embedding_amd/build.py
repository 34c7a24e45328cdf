"""Build librope_mi355x.so in-tree.

Host-only sources (contracts, C entry points) are compiled with g++; the HIP
kernels with hipcc for gfx950, -O3, IEEE arithmetic (no fast-math, f32
denormals kept), packed-fp32 instruction selection disabled; hipcc links.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librope_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["rope_plan.cpp", "rope_abi.cpp"]
# the kernels of each storage type in translation units of their own (the
# vector kernel; the row, scalar and table kernels), so that they compile in
# parallel
HIP_SOURCES = ["rope_kernels.hip",
               "rope_kernels_f32.hip", "rope_kernels_f16.hip", "rope_kernels_bf16.hip",
               "rope_kernels_f32_row.hip", "rope_kernels_f16_row.hip", "rope_kernels_bf16_row.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE,
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)

    def hip_obj(src):
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, "--offload-arch=" + ARCH, "-std=c++17", "-O3", "-fPIC", "-Wall", "-ffp-contract=off",
              "-fno-gpu-flush-denormals-to-zero",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    jobs = max(1, min(len(HIP_SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs += list(pool.map(hip_obj, HIP_SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv or True))
